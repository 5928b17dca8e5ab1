// Drives the library through its C ABI alone: host arrays read from files, device buffers
// from hipMalloc, one hipStream_t, no Python or torch. tests/test_gpu_capi.py writes the
// inputs, runs this program as a child process and checks what it writes against the oracle.
//
//   capi_driver DIR M K N GROUP
//     reads  DIR/w.f32 (fp32 [K, N]) and DIR/x.f16 (fp16 bits [M, K])
//     writes DIR/qweight.i32, scales.f16, zeros.f16   w4a16_pack
//            DIR/codes.u8, deq.f16                     w4a16_dequant (device)
//            DIR/y.f16                                 w4a16_matmul
//            DIR/y_noalloc.f16                         w4a16_matmul_noalloc
//            DIR/y_grouped0.f16, y_grouped1.f16        w4a16_matmul_grouped (the matrix twice,
//                                                      the second with its own x = x negated)
//            DIR/xq.u8, sx.f32, y8.f16                 w4a8_quantize_activations + w4a8_matmul
//                                                      (GROUP 128 or 256 only)
//     and checks that a misaligned x is refused with W4A16_ERR_ALIGNMENT before any launch.
// Exit status 0 on success; otherwise the failing call and w4a16_last_error_detail() on stderr.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "w4a16.h"

namespace {

std::string g_dir;

template <typename T>
std::vector<T> read_file(const char* name, size_t count) {
    std::vector<T> v(count);
    const std::string path = g_dir + "/" + name;
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f || std::fread(v.data(), sizeof(T), count, f) != count) {
        std::fprintf(stderr, "cannot read %zu elements from %s\n", count, path.c_str());
        std::exit(2);
    }
    std::fclose(f);
    return v;
}

template <typename T>
void write_file(const char* name, const std::vector<T>& v) {
    const std::string path = g_dir + "/" + name;
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f || std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) {
        std::fprintf(stderr, "cannot write %s\n", path.c_str());
        std::exit(2);
    }
    std::fclose(f);
}

void check(int rc, const char* what) {
    if (rc != W4A16_OK) {
        std::fprintf(stderr, "%s failed: %d %s: %s\n", what, rc, w4a16_strerror(rc), w4a16_last_error_detail());
        std::exit(1);
    }
}

void hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        std::exit(1);
    }
}

template <typename T>
T* device_copy(const std::vector<T>& h) {
    T* d = nullptr;
    hip_check(hipMalloc(reinterpret_cast<void**>(&d), h.size() * sizeof(T)), "hipMalloc");
    hip_check(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy to device");
    return d;
}

template <typename T>
T* device_alloc(size_t count) {
    T* d = nullptr;
    hip_check(hipMalloc(reinterpret_cast<void**>(&d), count * sizeof(T)), "hipMalloc");
    return d;
}

template <typename T>
std::vector<T> host_copy(const T* d, size_t count) {
    std::vector<T> h(count);
    hip_check(hipMemcpy(h.data(), d, count * sizeof(T), hipMemcpyDeviceToHost), "hipMemcpy to host");
    return h;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 6) {
        std::fprintf(stderr, "usage: %s DIR M K N GROUP\n", argv[0]);
        return 2;
    }
    g_dir = argv[1];
    const int64_t M = std::atoll(argv[2]), K = std::atoll(argv[3]), N = std::atoll(argv[4]), G = std::atoll(argv[5]);
    std::printf("capi_driver: M=%lld K=%lld N=%lld group=%lld, library version %d\n", (long long)M, (long long)K,
                (long long)N, (long long)G, (int)w4a16_version());

    const std::vector<float> w = read_file<float>("w.f32", (size_t)(K * N));
    const std::vector<uint16_t> x = read_file<uint16_t>("x.f16", (size_t)(M * K));

    // host packer
    std::vector<int32_t> qw((size_t)(K / 8 * N));
    std::vector<uint16_t> sc((size_t)(K / G * N)), zr((size_t)(K / G * N));
    check(w4a16_pack(w.data(), K, N, G, qw.data(), sc.data(), zr.data()), "w4a16_pack");
    write_file("qweight.i32", qw);
    write_file("scales.f16", sc);
    write_file("zeros.f16", zr);

    hipStream_t st;
    hip_check(hipStreamCreate(&st), "hipStreamCreate");
    uint16_t* dx = device_copy(x);
    std::vector<uint16_t> xneg(x);
    for (auto& h : xneg) h ^= 0x8000u;                     // -x, a second input for the grouped call
    uint16_t* dxneg = device_copy(xneg);
    int32_t* dqw = device_copy(qw);
    uint16_t* ds = device_copy(sc);
    uint16_t* dz = device_copy(zr);
    const size_t MN = (size_t)(M * N);
    uint16_t* dy = device_alloc<uint16_t>(MN);
    uint16_t* dy_na = device_alloc<uint16_t>(MN);
    uint16_t* dy_g0 = device_alloc<uint16_t>(MN);
    uint16_t* dy_g1 = device_alloc<uint16_t>(MN);
    uint8_t* dcodes = device_alloc<uint8_t>((size_t)(K * N));
    uint16_t* ddeq = device_alloc<uint16_t>((size_t)(K * N));

    check(w4a16_dequant(dqw, ds, dz, dcodes, ddeq, N, K, G, st), "w4a16_dequant");
    check(w4a16_matmul(dx, dqw, ds, dz, dy, M, N, K, G, st), "w4a16_matmul");
    check(w4a16_matmul_noalloc(dx, dqw, ds, dz, dy_na, M, N, K, G, W4A16_LAYOUT_LINEAR, st, nullptr),
          "w4a16_matmul_noalloc");
    const w4a16_matrix_t mats[2] = {{dqw, ds, dz, dy_g0, N, nullptr, 0}, {dqw, ds, dz, dy_g1, N, dxneg, 0}};
    check(w4a16_matmul_grouped(dx, mats, 2, M, K, G, W4A16_LAYOUT_LINEAR, st, nullptr), "w4a16_matmul_grouped");

    // an argument error is reported before anything is enqueued
    const int bad = w4a16_matmul(reinterpret_cast<const char*>(dx) + 2, dqw, ds, dz, dy, M, N, K, G, st);
    if (bad != W4A16_ERR_ALIGNMENT) {
        std::fprintf(stderr, "misaligned x: expected W4A16_ERR_ALIGNMENT, got %d\n", bad);
        return 1;
    }

    const bool w4a8 = G == 128 || G == 256;
    uint8_t* dxq = nullptr;
    float* dsx = nullptr;
    uint16_t* dy8 = nullptr;
    if (w4a8) {
        const int64_t Ms = (M + 3) / 4 * 4;
        dxq = device_alloc<uint8_t>((size_t)(M * K));
        dsx = device_alloc<float>((size_t)M);
        float* dxsum = device_alloc<float>((size_t)(K / 128 * Ms));
        dy8 = device_alloc<uint16_t>(MN);
        check(w4a8_quantize_activations(dx, dxq, dsx, dxsum, M, K, st), "w4a8_quantize_activations");
        check(w4a8_matmul(dxq, dsx, dxsum, dqw, ds, dz, dy8, M, N, K, G, W4A16_LAYOUT_LINEAR, st), "w4a8_matmul");
    }
    hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");

    write_file("codes.u8", host_copy(dcodes, (size_t)(K * N)));
    write_file("deq.f16", host_copy(ddeq, (size_t)(K * N)));
    write_file("y.f16", host_copy(dy, MN));
    write_file("y_noalloc.f16", host_copy(dy_na, MN));
    write_file("y_grouped0.f16", host_copy(dy_g0, MN));
    write_file("y_grouped1.f16", host_copy(dy_g1, MN));
    if (w4a8) {
        write_file("xq.u8", host_copy(dxq, (size_t)(M * K)));
        write_file("sx.f32", host_copy(dsx, (size_t)M));
        write_file("y8.f16", host_copy(dy8, MN));
    }
    hip_check(hipStreamDestroy(st), "hipStreamDestroy");
    std::printf("capi_driver: done\n");
    return 0;
}
