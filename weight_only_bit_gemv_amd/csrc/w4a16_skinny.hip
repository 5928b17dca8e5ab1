// Launch-side dispatch of the decode / skinny-M kernel over its built configurations (the
// kernel itself is in w4a16_skinny.hpp; each strip width is compiled in its own file).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "w4a16_internal.h"

namespace w4a16 {

bool skinny_config_supported(int row_tiles, int waves, int lw, int seg, int seg_group) {
    if (lw != 1 && lw != 2 && lw != 4) return false;
    if (seg != 1 && seg != 2 && seg != 4 && seg != 8) return false;
    // built (segment, K-steps of one group in it) pairs: every segment inside one group,
    // 4-step segments over 2 or 4 groups (64- and 32-row groups), 8-step over 2 groups
    if (!(seg_group == seg || (seg == 4 && (seg_group == 1 || seg_group == 2)) ||
          (seg == 2 && seg_group == 1) || (seg == 8 && seg_group == 4)))
        return false;
    if (seg == 8 && seg_group == 8) return false;
    if (waves != 4 && waves != 8 && waves != 16) return false;
    if (row_tiles < 1 || row_tiles > (lw == 4 ? 4 : 2)) return false;
    // built (row_tiles, waves) pairs: the LDS of the wave reduction, (waves - 1) * 16 *
    // row_tiles rows of 16 * lw floats, stays within 64 KiB, and register use stays low
    // enough for at least two work-groups' worth of waves per compute unit
    if (row_tiles >= 3 && waves != 4) return false;
    if (row_tiles == 2 && waves == 16) return false;
    return (waves - 1) * 16 * row_tiles * 16 * lw * 4 <= 64 * 1024;
}

int launch_skinny(const SkinnyParams& p, void* stream) {
    const int seg_group = std::min(p.seg, 1 << p.gshift);
    if ((p.kc % p.seg) != 0 || !skinny_config_supported(p.row_tiles, p.waves, p.lw, p.seg, seg_group))
        return (int)hipErrorInvalidValue;
    if (p.lw == 1) return launch_skinny_lw1(p, stream);
    if (p.lw == 2) return launch_skinny_lw2(p, stream);
    return launch_skinny_lw4(p, stream);
}

}  // namespace w4a16
