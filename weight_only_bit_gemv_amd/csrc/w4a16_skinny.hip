// Launch-side dispatch of the decode / skinny-M kernel over its built configurations (the
// kernel itself is in w4a16_skinny.hpp; each strip width is compiled in its own file).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "w4a16_internal.h"

namespace w4a16 {

int launch_skinny(const SkinnyParams& p, void* stream) {
    const int seg_group = std::min(p.seg, 1 << p.gshift);
    if ((p.kc % p.seg) != 0 || !skinny_config_supported(p.row_tiles, p.waves, p.lw, p.seg, seg_group))
        return (int)hipErrorInvalidValue;
    if (p.lw == 1) return launch_skinny_lw1(p, stream);
    if (p.lw == 2) return launch_skinny_lw2(p, stream);
    return launch_skinny_lw4(p, stream);
}

}  // namespace w4a16
