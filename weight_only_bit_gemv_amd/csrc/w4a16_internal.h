// Internal declarations shared by the C ABI layer, the host packer and the kernel launchers.
#pragma once

#include <cstdint>

#include "w4a16.h"

namespace w4a16 {

// ---- host packer (w4a16_pack.cpp) ----
uint16_t f32_to_f16_rne(float f);
float f16_to_f32(uint16_t h);
// K offset held by nibble p of a packed word, per W4A16_LAYOUT_*.
constexpr int kNibbleK[2][8] = {{0, 1, 2, 3, 4, 5, 6, 7}, {0, 2, 4, 6, 1, 3, 5, 7}};
inline bool layout_supported(int layout) {
    return layout == W4A16_LAYOUT_LINEAR || layout == W4A16_LAYOUT_INTERLEAVED;
}
int pack_host(const float* W, int64_t K, int64_t N, int64_t g, bool symmetric, int layout,
              int32_t* qweight, uint16_t* scales, uint16_t* zeros);
void unpack_host(const int32_t* qweight, int64_t K, int64_t N, int layout, uint8_t* codes);

// ---- decode / skinny kernel (w4a16_skinny.hip) ----
constexpr int kKStep = 32;           // K rows per MFMA step (4 packed rows)
// Supported group sizes: 32, 64, 128, 256 rows (1, 2, 4, 8 K-steps).
inline bool group_supported(int64_t g) { return g == 32 || g == 64 || g == 128 || g == 256; }
inline int log2_exact(int64_t v) { int r = 0; while ((int64_t(1) << r) < v) ++r; return r; }

// One weight matrix of a skinny launch. A launch covers 1..kMaxGroupMats matrices that share
// M, K, the group size, the layout and the plan (each with its own activations x, which may
// be the same buffer); their column strips are numbered one after the other: matrix i owns
// strips strip0 .. strip0 + ceil(N / cols) - 1.
constexpr int kMaxGroupMats = 16;
struct SkinnyMatrix {
    const uint16_t* x;        // fp16 [M, K]
    const uint32_t* qweight;  // int32 [K/8, N]
    const uint16_t* scales;   // fp16 [K/g, N]
    const uint16_t* zeros;    // fp16 [K/g, N]
    uint16_t* y;              // fp16 [M, N]
    int N;
    int strip0;               // first strip of this matrix
};

// The scalar arguments of a skinny launch.
struct SkinnyHeader {
    const uint16_t* x;        // fp16 [M, K] of a single-matrix launch (a grouped one reads mat[i].x)
    float* ws;                // fp32 partials [row_blocks][n_strips][splits][16*row_tiles][cols]
    uint32_t* counters;       // arrival counters [row_blocks][n_strips], zero between calls
    int M, K;
    int kc;                   // K-steps per wavefront
    int splits;               // work-groups along K per strip
    int n_strips;             // strips of all matrices: sum of ceil(N_i / cols)
    int row_tiles;            // 16-row tiles per work-group (1..4)
    int row_blocks;           // ceil(M / (16 * row_tiles))
    int waves;                // wavefronts per work-group (4, 8 or 16), each on its own K range
    int lw;                   // packed words per lane per K-step (1, 2, 4): cols = 16 * lw
    int seg;                  // K-steps per software-pipeline segment (1, 2, 4, 8)
    int gshift;               // log2(K-steps per scale/zero group): group of K-step ks = ks >> gshift
    int layout;               // W4A16_LAYOUT_*
    int n_mats;               // matrices in this launch (1 for w4a16_matmul)
};

// Kernel arguments, by launch kind GM (each kind is its own kernel instance; sharing one
// argument block between them measured slower per launch):
//   GM = 1               a single matrix: one small contiguous block, x in the header (a
//                        16-entry table made every 4096 x 4096 GEMV 0.15 us slower);
//   GM = kSharedXMats    up to 4 matrices that share the header's x (q/k/v, gate/up);
//   GM = kMaxGroupMats   up to 16 matrices, each with its own x and row count (mixture-of-experts
//                        layers):
//                        the entries' first strips side by side, then the table. Against
//                        the 4-entry kind this costs 0.2 us (x from the entry) + 0.3 us (16
//                        entries) per launch on q/k/v.
constexpr int kSharedXMats = 4;
template <int GM>
struct SkinnyArgs : SkinnyHeader {
    SkinnyMatrix mat[GM];
};
template <>
struct SkinnyArgs<kMaxGroupMats> : SkinnyHeader {
    int strip0[kMaxGroupMats];   // mat[i].strip0
    int rows[kMaxGroupMats];     // rows of matrix i's x and y (<= M; the grid covers M)
    SkinnyMatrix mat[kMaxGroupMats];
};
typedef SkinnyArgs<kMaxGroupMats> SkinnyParams;   // as the host fills them

// Workspace a skinny launch needs (bytes of partials, number of counters).
inline void skinny_workspace(const SkinnyParams& p, uint64_t* ws_bytes, uint64_t* n_counters) {
    if (p.splits <= 1) { *ws_bytes = 0; *n_counters = 0; return; }
    *ws_bytes = (uint64_t)p.row_blocks * p.n_strips * p.splits * 16ull * p.row_tiles * 16ull * p.lw * 4ull;
    *n_counters = (uint64_t)p.row_blocks * p.n_strips;
}

int launch_skinny(const SkinnyParams& p, void* stream);   // returns a hipError_t value
// seg_group = min(seg, K-steps per group): K-steps of one group inside a segment.
bool skinny_config_supported(int row_tiles, int waves, int lw, int seg, int seg_group);
// per strip width (w4a16_skinny_lw{1,2,4}.hip); hipErrorInvalidValue for a config not built
int launch_skinny_lw1(const SkinnyParams& p, void* stream);
int launch_skinny_lw2(const SkinnyParams& p, void* stream);
int launch_skinny_lw4(const SkinnyParams& p, void* stream);

// ---- prefill kernel (w4a16_prefill.hip) ----
constexpr int kPrefillBM = 128;      // rows of M per work-group
constexpr int kPrefillBN = 128;      // columns per work-group

struct PrefillParams {
    const uint16_t* x;        // fp16 [M, K]
    const uint32_t* qweight;  // int32 [K/8, N]
    const uint16_t* scales;   // fp16 [K/g, N]
    const uint16_t* zeros;    // fp16 [K/g, N]
    uint16_t* y;              // fp16 [M, N]
    int M, N, K;
    int tile;                 // W4A16_TILE_LDS, W4A16_TILE_REGISTER_B or W4A16_TILE_ASYNC
    int group_shift;          // log2(rows per scale/zero group)
    int layout;               // W4A16_LAYOUT_*
    int bm;                   // W4A16_TILE_ASYNC: rows of M per work-group, 32, 64 or 128
    // split-K (W4A16_TILE_ASYNC only): work-groups along K per output tile, each over
    // stages_per_split 64-row stages (the last over the rest, >= 2); fp32 partials of
    // up to 128 x 256 per (tile, split) in ws, arrival counters per tile (zero between calls)
    int splits;
    int stages_per_split;
    float* ws;
    uint32_t* counters;
};

constexpr int kPrefillTileFloats = 128 * 256;   // one fp32 partial of the async tile

int launch_prefill(const PrefillParams& p, void* stream);  // returns a hipError_t value
int launch_prefill_rb(const PrefillParams& p, void* stream);  // W4A16_TILE_REGISTER_B (w4a16_prefill_rb.hip)
int launch_prefill_async(const PrefillParams& p, void* stream);  // W4A16_TILE_ASYNC (w4a16_prefill_async.hip)

// ---- W4A8: E4M3 activations x 4-bit weights (w4a8_prefill.hip) ----
struct W4A8Params {
    const uint8_t* xq;        // E4M3 codes [M, K]
    const float* sx;          // fp32 row scales [M]
    const float* xsum;        // fp32 block sums of the decoded codes [K/128, Ms]
    int Ms;                   // row stride of xsum: M rounded up to a multiple of 4
    const uint32_t* qweight;  // int32 [K/8, N]
    const uint16_t* scales;   // fp16 [K/g, N]
    const uint16_t* zeros;    // fp16 [K/g, N]
    uint16_t* y;              // fp16 [M, N]
    int M, N, K;
    int group_shift;          // log2(rows per group): 7 or 8
    int layout;               // W4A16_LAYOUT_*
    int bm;                   // rows of M per work-group: 32, 64 or 128
    // split-K as on the async W4A16 tile: work-groups along K per output tile, each over
    // stages_per_split 128-row stages (the last over the rest, >= 1); fp32 partials of
    // up to 128 x 256 per (tile, split) in ws, arrival counters per tile (zero between calls)
    int splits;
    int stages_per_split;
    float* ws;
    uint32_t* counters;
};
int launch_w4a8_quantize(const uint16_t* x, uint8_t* xq, float* sx, float* xsum, int M, int K, void* stream);
int launch_w4a8(const W4A8Params& p, void* stream);   // returns a hipError_t value

// ---- static scratch of w4a16_matmul_noalloc (w4a16_noalloc.hip) ----
constexpr uint64_t kScratchCounterBytes = 256ull << 10;   // 65536 arrival counters
constexpr uint64_t kScratchPartialBytes = 64ull << 20;    // fp32 split-K partials
// Device addresses of this device's counters and partials (the counters are cleared on the
// device's first call, by a kernel on `stream`). Returns a hipError_t value.
int scratch_workspace(void* stream, float** partials, uint32_t** counters);

// ---- read probe (w4a16_readbw.hip) ----
int launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

// ---- dequant hook (w4a16_dequant.hip) ----
int launch_dequant(const uint32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                   uint8_t* codes, uint16_t* w, int N, int K, int group_shift, int layout, void* stream);

}  // namespace w4a16
