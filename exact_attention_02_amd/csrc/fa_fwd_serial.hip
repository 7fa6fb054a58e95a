// Launch of the serial forward kernel (fa_serial.h): picks the instantiation
// set for the input type and the score modifier. Each set is compiled in an
// object of its own from fa_fwd_serial_inst.hip.
#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace fa {

int launch_serial(const Plan& pl, const Params& p, void* stream) {
    if (pl.nw != 4 && pl.nw != 8) return (int)hipErrorInvalidValue;
    if (pl.in == IN_F16) {
        if (p.mod == MOD_NONE) return launch_serial_in<IN_F16, MOD_NONE>(pl, p, stream);
        if (p.mod == MOD_SOFTCAP) return launch_serial_in<IN_F16, MOD_SOFTCAP>(pl, p, stream);
        if (p.mod == MOD_ALIBI) return launch_serial_in<IN_F16, MOD_ALIBI>(pl, p, stream);
    }
    if (pl.in == IN_E4M3 && p.mod == MOD_NONE) return launch_serial_in<IN_E4M3, MOD_NONE>(pl, p, stream);
    if (pl.in == IN_BF16) {
        if (p.mod == MOD_NONE) return launch_serial_in<IN_BF16, MOD_NONE>(pl, p, stream);
        if (p.mod == MOD_SOFTCAP) return launch_serial_in<IN_BF16, MOD_SOFTCAP>(pl, p, stream);
        if (p.mod == MOD_ALIBI) return launch_serial_in<IN_BF16, MOD_ALIBI>(pl, p, stream);
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace fa
