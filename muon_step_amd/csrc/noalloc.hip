// Fixed device scratch of the allocation-free variant of muon_step, for
// callers that cannot allocate device memory during a step (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// One static array per GPU the library runs on, held until the process ends.
// In host code the name `scratch` is only a host-side stand-in: the device
// address of each GPU's copy comes from hipGetSymbolAddress, called once per
// device by muon_create with that device current, and only that address is
// ever handed to kernels or copies.
#include "kernels.hpp"

static __device__ __align__(256) char scratch[muon::kScratchBytes];

namespace muon {

hipError_t scratch_address(void **out) { return hipGetSymbolAddress(out, HIP_SYMBOL(scratch)); }

}  // namespace muon
