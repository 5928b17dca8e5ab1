// Decode / skinny-M kernel instances with 16-column strips (4-byte weight loads per lane).
#include <algorithm>

#include "w4a16_skinny.hpp"

namespace w4a16 {

int launch_skinny_lw1(const SkinnyParams& p, void* stream) {
    using namespace skinny;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int sg = std::min(p.seg, 1 << p.gshift);
#define W4A16_CASE(MT, U, SG, W) \
    if (p.row_tiles == MT && p.seg == U && sg == SG && p.waves == W) return (int)launch_one<MT, 1, U, SG, W>(p, s);
#define W4A16_SEGS(MT, W) W4A16_CASE(MT, 1, 1, W) W4A16_CASE(MT, 2, 1, W) W4A16_CASE(MT, 2, 2, W) \
    W4A16_CASE(MT, 4, 1, W) W4A16_CASE(MT, 4, 2, W) W4A16_CASE(MT, 4, 4, W) W4A16_CASE(MT, 8, 4, W)
    W4A16_SEGS(1, 4) W4A16_SEGS(1, 8) W4A16_SEGS(1, 16)
    W4A16_SEGS(2, 4) W4A16_SEGS(2, 8)
#undef W4A16_SEGS
#undef W4A16_CASE
    return (int)hipErrorInvalidValue;
}

}  // namespace w4a16
