// Decode / skinny-M kernel instances with 32-column strips (8-byte weight loads per lane).
#include "w4a16_skinny.hpp"

namespace w4a16 {

int launch_skinny_lw2(const SkinnyParams& p, void* stream) {
    using namespace skinny;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define W4A16_CASE(MT, U, W) \
    if (p.row_tiles == MT && p.seg == U && p.waves == W) return (int)launch_one<MT, 2, U, W>(p, s);
#define W4A16_SEGS(MT, W) W4A16_CASE(MT, 1, W) W4A16_CASE(MT, 2, W) W4A16_CASE(MT, 4, W) W4A16_CASE(MT, 8, W)
    W4A16_SEGS(1, 4) W4A16_SEGS(1, 8) W4A16_SEGS(1, 16)
    W4A16_SEGS(2, 4) W4A16_SEGS(2, 8)
#undef W4A16_SEGS
#undef W4A16_CASE
    return (int)hipErrorInvalidValue;
}

}  // namespace w4a16
