// Host-side stand-ins for the kernel launchers of libseed, for the sanitizer build of the C ABI
// (tests/c/abi_validate.c). Every launcher counts its calls and returns success without touching
// device memory: a call that reaches one is a call the ABI accepted. The support queries accept
// what the library compiles (d_k, d_v in {64, 128} is checked by the ABI itself).
#include <hip/hip_runtime.h>

#include "../../include/seed.h"
#include "../../rank_recurrent_state_amd/csrc/kernels.hpp"

extern "C" {
int seed_stub_launches = 0;
}

namespace seed {
namespace {
hipError_t counted() {
  ++seed_stub_launches;
  return hipSuccess;
}
}  // namespace
hipError_t launch_decode(const seed_shape&, const StepArgs&, hipStream_t) { return counted(); }
hipError_t launch_dense(const seed_shape&, const DenseArgs&, hipStream_t) { return counted(); }
hipError_t launch_compress(const seed_shape&, const CompressArgs&, hipStream_t) { return counted(); }
hipError_t launch_from_dense(const seed_shape&, const CompressArgs&, hipStream_t) { return counted(); }
hipError_t launch_energy(const seed_shape&, const EnergyArgs&, hipStream_t) { return counted(); }
hipError_t launch_decode_chunk(const seed_shape&, const StepArgs&, hipStream_t) { return counted(); }
hipError_t launch_spectrum(const seed_shape&, const CompressArgs&, hipStream_t) { return counted(); }
int32_t chunk_max_tokens() { return 32; }
bool decode_supported(const seed_shape&) { return true; }
bool compress_supported(const seed_shape&) { return true; }
bool chunk_supported(const seed_shape&) { return true; }
bool chunk_supported_len(const seed_shape& sh, int32_t len) { return sh.kind != SEED_KDA || len <= 16; }
int32_t from_dense_iterations() { return 30; }
}  // namespace seed
