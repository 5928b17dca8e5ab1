// Host driver for the sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer) of the
// W4A16 packer and of the C ABI's validation and dispatch layer. Built with g++ alone: the
// HIP runtime and the kernel launchers are replaced by stubs that abort, so every call made
// here must be settled (done or rejected) before any HIP call.
//
//   host_driver <dir>   packs every case listed in <dir>/cases.txt ("K N group symmetric
//                       layout" per line; W in w<i>.bin as raw fp32), writes q<i>.bin,
//                       s<i>.bin, z<i>.bin and c<i>.bin (codes from w4a16_unpack_ex), then
//                       runs the error-path and plan checks and prints "checks ok <n>".
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "w4a16_internal.h"

[[noreturn]] static void reached(const char* what) {
    std::fprintf(stderr, "HIP call reached in a host-only run: %s\n", what);
    std::abort();
}

extern "C" {
hipError_t hipGetDevice(int*) { reached("hipGetDevice"); }
const char* hipGetErrorString(hipError_t) { reached("hipGetErrorString"); }
hipError_t hipMalloc(void**, size_t) { reached("hipMalloc"); }
hipError_t hipFree(void*) { reached("hipFree"); }
hipError_t hipMemsetAsync(void*, int, size_t, hipStream_t) { reached("hipMemsetAsync"); }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus*) { reached("hipStreamIsCapturing"); }
hipError_t hipStreamSynchronize(hipStream_t) { reached("hipStreamSynchronize"); }
hipError_t hipStreamCreateWithFlags(hipStream_t*, unsigned int) { reached("hipStreamCreateWithFlags"); }
hipError_t hipStreamDestroy(hipStream_t) { reached("hipStreamDestroy"); }
hipError_t hipStreamBeginCapture(hipStream_t, hipStreamCaptureMode) { reached("hipStreamBeginCapture"); }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t*) { reached("hipStreamEndCapture"); }
hipError_t hipGraphInstantiate(hipGraphExec_t*, hipGraph_t, hipGraphNode_t*, char*, size_t) {
    reached("hipGraphInstantiate");
}
hipError_t hipGraphLaunch(hipGraphExec_t, hipStream_t) { reached("hipGraphLaunch"); }
hipError_t hipGraphExecDestroy(hipGraphExec_t) { reached("hipGraphExecDestroy"); }
hipError_t hipGraphDestroy(hipGraph_t) { reached("hipGraphDestroy"); }
hipError_t hipEventCreate(hipEvent_t*) { reached("hipEventCreate"); }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { reached("hipEventRecord"); }
hipError_t hipEventSynchronize(hipEvent_t) { reached("hipEventSynchronize"); }
hipError_t hipEventElapsedTime(float*, hipEvent_t, hipEvent_t) { reached("hipEventElapsedTime"); }
hipError_t hipEventDestroy(hipEvent_t) { reached("hipEventDestroy"); }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { reached("hipMemcpyAsync"); }
}

namespace w4a16 {
int launch_skinny(const SkinnyParams&, void*) { reached("launch_skinny"); }
int launch_prefill(const PrefillParams&, void*) { reached("launch_prefill"); }
int launch_dequant(const uint32_t*, const uint16_t*, const uint16_t*, uint8_t*, uint16_t*, int, int, int, int,
                   void*) {
    reached("launch_dequant");
}
int launch_w4a8_quantize(const uint16_t*, uint8_t*, float*, float*, int, int, void*) {
    reached("launch_w4a8_quantize");
}
int launch_w4a8(const W4A8Params&, void*) { reached("launch_w4a8"); }
int scratch_workspace(void*, float**, uint32_t**) { reached("scratch_workspace"); }
int launch_read_probe(const void*, int64_t, uint32_t*, void*) { reached("launch_read_probe"); }
}  // namespace w4a16

static int g_checks = 0;
static int g_failed = 0;

static void expect(int got, int want, const char* what) {
    ++g_checks;
    if (got != want) {
        ++g_failed;
        std::fprintf(stderr, "FAIL %s: got %d, want %d (%s)\n", what, got, want, w4a16_last_error_detail());
    }
}

template <class T>
static std::vector<T> read_file(const std::string& path, size_t n) {
    std::vector<T> v(n);
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f || std::fread(v.data(), sizeof(T), n, f) != n) {
        std::fprintf(stderr, "cannot read %s\n", path.c_str());
        std::exit(2);
    }
    std::fclose(f);
    return v;
}

template <class T>
static void write_file(const std::string& path, const std::vector<T>& v) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f || std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) {
        std::fprintf(stderr, "cannot write %s\n", path.c_str());
        std::exit(2);
    }
    std::fclose(f);
}

static void pack_cases(const std::string& dir) {
    FILE* f = std::fopen((dir + "/cases.txt").c_str(), "r");
    if (!f) {
        std::fprintf(stderr, "no cases.txt\n");
        std::exit(2);
    }
    long long K, N, g;
    int sym, layout, i = 0;
    while (std::fscanf(f, "%lld %lld %lld %d %d", &K, &N, &g, &sym, &layout) == 5) {
        const std::string id = std::to_string(i++);
        std::vector<float> W = read_file<float>(dir + "/w" + id + ".bin", (size_t)(K * N));
        std::vector<int32_t> q((size_t)(K / 8 * N));
        std::vector<uint16_t> s((size_t)(K / g * N)), z((size_t)(K / g * N));
        std::vector<uint8_t> c((size_t)(K * N));
        expect(w4a16_pack_ex(W.data(), K, N, g, sym, layout, q.data(), s.data(), z.data()), W4A16_OK, "pack case");
        expect(w4a16_unpack_ex(q.data(), K, N, layout, c.data()), W4A16_OK, "unpack case");
        write_file(dir + "/q" + id + ".bin", q);
        write_file(dir + "/s" + id + ".bin", s);
        write_file(dir + "/z" + id + ".bin", z);
        write_file(dir + "/c" + id + ".bin", c);
    }
    std::fclose(f);
}

static void pack_errors() {
    const int64_t K = 256, N = 12;
    std::vector<float> W((size_t)(K * N), 0.01f);
    for (size_t i = 0; i < W.size(); ++i) W[i] = 0.01f * (float)((i * 37) % 23) - 0.1f;
    std::vector<int32_t> q((size_t)(K / 8 * N));
    std::vector<uint16_t> s((size_t)(K / 32 * N)), z((size_t)(K / 32 * N));
    expect(w4a16_pack(nullptr, K, N, 128, q.data(), s.data(), z.data()), W4A16_ERR_INVALID_ARG, "pack null W");
    expect(w4a16_pack(W.data(), K, N, 128, nullptr, s.data(), z.data()), W4A16_ERR_INVALID_ARG, "pack null q");
    expect(w4a16_pack(W.data(), 0, N, 128, q.data(), s.data(), z.data()), W4A16_ERR_INVALID_ARG, "pack K=0");
    expect(w4a16_pack(W.data(), K, -3, 128, q.data(), s.data(), z.data()), W4A16_ERR_INVALID_ARG, "pack N<0");
    expect(w4a16_pack(W.data(), K, N, 48, q.data(), s.data(), z.data()), W4A16_ERR_UNSUPPORTED, "pack g=48");
    expect(w4a16_pack(W.data(), 192, N, 128, q.data(), s.data(), z.data()), W4A16_ERR_UNSUPPORTED, "pack K%g");
    expect(w4a16_pack_ex(W.data(), K, N, 128, 2, 0, q.data(), s.data(), z.data()), W4A16_ERR_INVALID_ARG,
           "pack symmetric=2");
    expect(w4a16_pack_ex(W.data(), K, N, 128, 0, 7, q.data(), s.data(), z.data()), W4A16_ERR_INVALID_ARG,
           "pack layout=7");
    std::vector<float> bad = W;
    bad[(size_t)(K * N - 1)] = std::nanf("");
    expect(w4a16_pack(bad.data(), K, N, 32, q.data(), s.data(), z.data()), W4A16_ERR_NONFINITE, "pack NaN");
    bad = W;
    bad[5] = -INFINITY;
    expect(w4a16_pack_ex(bad.data(), K, N, 32, 1, 1, q.data(), s.data(), z.data()), W4A16_ERR_NONFINITE, "pack -Inf");
    bad = W;
    bad[0] = -1.0e6f;
    bad[(size_t)N] = 1.0e6f;                                   // range/15 > 65504: fp16 scale overflow
    expect(w4a16_pack(bad.data(), K, N, 32, q.data(), s.data(), z.data()), W4A16_ERR_NONFINITE, "pack scale overflow");
    bad.assign(W.size(), 1000.0f);
    bad[0] = 1000.0625f;                                       // one-signed group: zero far below -1024
    expect(w4a16_pack(bad.data(), K, N, 32, q.data(), s.data(), z.data()), W4A16_ERR_UNSUPPORTED, "pack |zero|>1024");
    std::vector<uint8_t> c((size_t)(K * N));
    expect(w4a16_unpack(nullptr, K, N, c.data()), W4A16_ERR_INVALID_ARG, "unpack null");
    expect(w4a16_unpack(q.data(), 4, N, c.data()), W4A16_ERR_INVALID_ARG, "unpack K=4");
    expect(w4a16_unpack_ex(q.data(), K, N, 3, c.data()), W4A16_ERR_INVALID_ARG, "unpack layout=3");
}

static void device_call_errors() {
    // fake 16-byte aligned addresses: never dereferenced, every call below is rejected first
    void* p[6];
    for (int i = 0; i < 6; ++i) p[i] = reinterpret_cast<void*>(uintptr_t(0x100000 + 0x1000 * i));
    void* mis = reinterpret_cast<void*>(uintptr_t(0x100008));
    auto mm = [&](int64_t M, int64_t N, int64_t K, int64_t g, void* a = nullptr) {
        return w4a16_matmul(a ? a : p[0], (const int32_t*)p[1], p[2], p[3], p[4], M, N, K, g, nullptr);
    };
    expect(w4a16_matmul(nullptr, (const int32_t*)p[1], p[2], p[3], p[4], 1, 64, 128, 128, nullptr),
           W4A16_ERR_INVALID_ARG, "matmul null x");
    expect(mm(0, 64, 128, 128), W4A16_ERR_INVALID_ARG, "matmul M=0");
    expect(mm(1, 0, 128, 128), W4A16_ERR_INVALID_ARG, "matmul N=0");
    expect(mm(1, 62, 128, 128), W4A16_ERR_UNSUPPORTED, "matmul N%4");
    expect(mm(1, 64, 100, 128), W4A16_ERR_UNSUPPORTED, "matmul K%128");
    expect(mm(1, 64, 128, 48), W4A16_ERR_UNSUPPORTED, "matmul g=48");
    expect(mm(1, 64, 128, 128, mis), W4A16_ERR_ALIGNMENT, "matmul misaligned x");
    expect(mm(1, int64_t(1) << 29, 1 << 10, 128), W4A16_ERR_UNSUPPORTED, "matmul too large");
    const w4a16_plan_t bad_plans[] = {
        {7, 0, 0, 0, 0, 0, 0, 0},  {1, 0, 0, 0, 0, 0, 24, 0}, {1, 0, 0, 5, 0, 0, 0, 0},
        {1, 3, 0, 0, 0, 0, 0, 0},  {1, 0, 0, 0, 0, 5, 0, 0},  {1, 4, 0, 0, 0, 4, 64, 3},
        {2, 0, 0, 0, 9, 0, 0, 0},  {2, 0, -1, 0, 3, 0, 0, 0}, {2, 4, 0, 0, 3, 0, 0, 0},
        {2, 0, 2, 0, 1, 0, 0, 0},  {1, 4, 3, 0, 0, 4, 16, 4},
    };
    for (const w4a16_plan_t& pl : bad_plans)
        expect(w4a16_matmul_ex(p[0], (const int32_t*)p[1], p[2], p[3], p[4], 1, 64, 1024, 128, nullptr, &pl),
               W4A16_ERR_INVALID_ARG, "matmul_ex bad plan");
    expect(w4a16_matmul_ex(p[0], (const int32_t*)p[1], p[2], p[3], p[4], 1, 64, 1024, 128, nullptr, nullptr),
           W4A16_ERR_INVALID_ARG, "matmul_ex null plan");
    expect(w4a16_matmul_fmt(p[0], (const int32_t*)p[1], p[2], p[3], p[4], 1, 64, 1024, 128, 2, nullptr, nullptr),
           W4A16_ERR_INVALID_ARG, "matmul_fmt layout=2");
    const w4a16_plan_t many_splits{2, 0, 64, 0, 3, 0, 0, 0};   // 64 tiles x 64 splits x 128 KiB > the scratch
    expect(w4a16_matmul_noalloc(p[0], (const int32_t*)p[1], p[2], p[3], p[4], 130, 8192, 8192, 128, 0, nullptr,
                                &many_splits),
           W4A16_ERR_UNSUPPORTED, "noalloc plan beyond the static scratch");
    expect(w4a16_matmul_noalloc(p[0], nullptr, p[2], p[3], p[4], 1, 64, 128, 128, 0, nullptr, nullptr),
           W4A16_ERR_INVALID_ARG, "noalloc null qweight");
    w4a16_matrix_t gm[17];
    for (int i = 0; i < 17; ++i)
        gm[i] = w4a16_matrix_t{(const int32_t*)p[1], p[2], p[3], p[4], 64, nullptr, 0};
    expect(w4a16_matmul_grouped(p[0], gm, 17, 1, 4096, 128, 0, nullptr, nullptr), W4A16_ERR_INVALID_ARG,
           "grouped 17 matrices");
    gm[1].x = mis;
    expect(w4a16_matmul_grouped(p[0], gm, 3, 1, 4096, 128, 0, nullptr, nullptr), W4A16_ERR_ALIGNMENT,
           "grouped misaligned own x");
    gm[1].x = p[0];
    gm[2].M = 2;                                        // more rows than the call's M = 1
    expect(w4a16_matmul_grouped(p[0], gm, 3, 1, 4096, 128, 0, nullptr, nullptr), W4A16_ERR_INVALID_ARG,
           "grouped M_i > M");
    gm[2].M = 0;
    expect(w4a16_matmul_grouped(p[0], gm, 0, 1, 4096, 128, 0, nullptr, nullptr), W4A16_ERR_INVALID_ARG,
           "grouped 0 matrices");
    gm[2].N = 62;
    expect(w4a16_matmul_grouped(p[0], gm, 3, 1, 4096, 128, 0, nullptr, nullptr), W4A16_ERR_UNSUPPORTED,
           "grouped N%4");
    gm[2].N = 64;
    gm[1].zeros = mis;
    expect(w4a16_matmul_grouped(p[0], gm, 3, 1, 4096, 128, 0, nullptr, nullptr), W4A16_ERR_ALIGNMENT,
           "grouped misaligned zeros");
    gm[1].zeros = p[3];
    expect(w4a16_matmul_grouped(p[0], gm, 3, 1, 4096, 100, 0, nullptr, nullptr), W4A16_ERR_UNSUPPORTED,
           "grouped g=100");
    w4a16_plan_t async{2, 0, 0, 0, 3, 0, 0, 0};
    expect(w4a16_matmul_ex(p[0], (const int32_t*)p[1], p[2], p[3], p[4], 1, 60, 1024, 128, nullptr, &async),
           W4A16_ERR_UNSUPPORTED, "async tile N%8");
    uint8_t* codes = reinterpret_cast<uint8_t*>(p[5]);
    expect(w4a16_dequant((const int32_t*)p[1], p[2], p[3], nullptr, nullptr, 64, 128, 128, nullptr),
           W4A16_ERR_INVALID_ARG, "dequant no outputs");
    expect(w4a16_dequant((const int32_t*)p[1], p[2], p[3], codes + 2, nullptr, 64, 128, 128, nullptr),
           W4A16_ERR_ALIGNMENT, "dequant misaligned codes");
    expect(w4a16_dequant_fmt((const int32_t*)p[1], p[2], p[3], codes, nullptr, 64, 128, 128, 4, nullptr),
           W4A16_ERR_INVALID_ARG, "dequant layout=4");
    float* xs = (float*)p[3];
    expect(w4a8_quantize_activations(p[0], (uint8_t*)p[1], (float*)p[2], xs, 4, 200, nullptr), W4A16_ERR_UNSUPPORTED,
           "w4a8 quantise K%128");
    expect(w4a8_quantize_activations(p[0], (uint8_t*)p[1], reinterpret_cast<float*>(uintptr_t(0x100002)), xs, 4, 256,
                                     nullptr),
           W4A16_ERR_ALIGNMENT, "w4a8 quantise misaligned sx");
    const uint8_t* xq = (const uint8_t*)p[0];
    const float* sx = (const float*)p[5];
    expect(w4a8_matmul(xq, sx, xs, (const int32_t*)p[1], p[2], p[3], p[4], 4, 64, 256, 64, 0, nullptr),
           W4A16_ERR_UNSUPPORTED, "w4a8 g=64");
    expect(w4a8_matmul(xq, sx, xs, (const int32_t*)p[1], p[2], p[3], p[4], 4, 60, 256, 128, 0, nullptr),
           W4A16_ERR_UNSUPPORTED, "w4a8 N%8");
    expect(w4a8_matmul_ex(xq, sx, xs, (const int32_t*)p[1], p[2], p[3], p[4], 1, int64_t(1) << 25, 128, 128, 0, 0,
                          nullptr),
           W4A16_ERR_UNSUPPORTED, "w4a8 weight offsets");
    expect(w4a8_matmul_ex(xq, sx, xs, (const int32_t*)p[1], p[2], p[3], p[4], 1, 8, int64_t(1) << 21, 128, 0, 16384,
                          nullptr),
           W4A16_ERR_UNSUPPORTED, "w4a8 workspace offsets");
    expect(w4a8_matmul_ex(xq, sx, xs, (const int32_t*)p[1], p[2], p[3], p[4], 4, 64, 256, 128, 0, 3, nullptr),
           W4A16_ERR_INVALID_ARG, "w4a8 splits > K/128");
    expect(w4a16_read_probe(p[0], 100, (uint32_t*)p[1], nullptr), W4A16_ERR_INVALID_ARG, "read probe bytes%16");
    expect(w4a16_read_probe(nullptr, 1024, (uint32_t*)p[1], nullptr), W4A16_ERR_INVALID_ARG, "read probe null");
    expect(w4a16_read_probe(mis, 1024, (uint32_t*)p[1], nullptr), W4A16_ERR_ALIGNMENT, "read probe misaligned");
    expect(w4a16_autotune(nullptr, (const int32_t*)p[1], p[2], p[3], p[4], 1, 64, 128, 128, 0, nullptr, nullptr,
                          nullptr),
           W4A16_ERR_INVALID_ARG, "autotune null x");
    expect(w4a16_autotune(p[0], (const int32_t*)p[1], p[2], p[3], mis, 1, 64, 128, 128, 0, nullptr, nullptr, nullptr),
           W4A16_ERR_ALIGNMENT, "autotune misaligned y");
    expect(w4a16_autotune(p[0], (const int32_t*)p[1], p[2], p[3], p[4], 1, 66, 128, 128, 0, nullptr, nullptr, nullptr),
           W4A16_ERR_UNSUPPORTED, "autotune N%4");
    {
        w4a16_plan_t none{}, bad{}, good{};
        bad.kernel = W4A16_KERNEL_SKINNY;
        bad.cols = 48;
        good.kernel = W4A16_KERNEL_SKINNY;
        good.cols = 32;
        good.waves = 8;
        expect(w4a16_set_plan(1, 4096, 4096, 128, &none), W4A16_ERR_INVALID_ARG, "set_plan names no kernel");
        expect(w4a16_set_plan(1, 4096, 4096, 128, &bad), W4A16_ERR_INVALID_ARG, "set_plan cols 48");
        expect(w4a16_set_plan(1, 4096, 4096, 128, &good), W4A16_OK, "set_plan");
        w4a16_plan_t got{};
        expect(w4a16_plan(1, 4096, 4096, 128, &got), W4A16_OK, "plan after set_plan");
        expect(got.cols == 32 && got.waves == 8, 1, "plan is the one set");
        expect(w4a16_set_plan(1, 4096, 4096, 128, nullptr), W4A16_OK, "set_plan remove");
        expect(w4a16_clear_plans(), W4A16_OK, "clear_plans");
    }
    for (int code = -7; code <= 1; ++code) {
        ++g_checks;
        if (!w4a16_strerror(code) || !*w4a16_strerror(code)) ++g_failed;
    }
}

static void plan_grid() {
    const int64_t Ms[] = {1, 2, 3, 4, 8, 15, 16, 17, 24, 31, 32, 33, 48, 63, 64, 65, 96, 127, 128, 129, 255, 512, 1000,
                          2048, 4096};
    const int64_t KNs[][2] = {{128, 4},      {128, 8},     {256, 100},  {384, 1412},  {768, 2048},  {1408, 2048},
                              {2048, 768},   {2048, 1408}, {4096, 4096}, {4096, 14336}, {14336, 4096}, {8192, 8192},
                              {8192, 28672}, {28672, 8192}, {4096, 128256}, {12288, 12}};
    const int64_t gs[] = {32, 64, 128, 256};
    for (int64_t M : Ms)
        for (const auto& kn : KNs)
            for (int64_t g : gs) {
                const int64_t K = kn[0], N = kn[1];
                if (K % g != 0) continue;
                w4a16_plan_t pl{};
                const int rc = w4a16_plan(M, N, K, g, &pl);
                expect(rc, W4A16_OK, "plan");
                if (rc) continue;
                ++g_checks;
                if (pl.kernel == W4A16_KERNEL_SKINNY) {
                    // the work-groups along K cover K: splits * waves * kc >= K / 32
                    if ((int64_t)pl.splits * pl.waves * pl.kc < K / 32 || pl.kc % pl.seg != 0) ++g_failed;
                } else if (pl.kernel == W4A16_KERNEL_PREFILL) {
                    if (pl.splits < 1 || pl.splits > K / 128 || (pl.tile == W4A16_TILE_ASYNC && N % 8 != 0)) ++g_failed;
                } else {
                    ++g_failed;
                }
            }
}

int main(int argc, char** argv) {
    if (argc > 1) pack_cases(argv[1]);
    pack_errors();
    device_call_errors();
    plan_grid();
    if (g_failed) {
        std::fprintf(stderr, "%d of %d checks failed\n", g_failed, g_checks);
        return 1;
    }
    std::printf("checks ok %d\n", g_checks);
    return 0;
}
