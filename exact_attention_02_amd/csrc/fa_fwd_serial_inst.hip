// One instantiation set of the serial forward kernel (fa_serial.h): the build
// compiles this file once per input type and score modifier, given as
// FA_SR_IN (InKind) and FA_SR_MOD (ScoreMod), so that the sets compile in
// parallel.
#include "fa_serial.h"

#if !defined(FA_SR_IN) || !defined(FA_SR_MOD)
#error "FA_SR_IN and FA_SR_MOD select the instantiation set"
#endif

namespace fa {

template int launch_serial_in<FA_SR_IN, FA_SR_MOD>(const Plan& pl, const Params& p, void* stream);

}  // namespace fa
