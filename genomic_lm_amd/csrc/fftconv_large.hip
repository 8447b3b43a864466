// fftconv_large.hip -- single-pass modal Hyena operator for L > 32768.
// Not implemented in this build: the size query reports 0 bytes and the entry
// point answers HYENA_ERR_UNSUPPORTED for these lengths.
#include "launch.hpp"

namespace hyena {

size_t fftconv_large_workspace(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_fftconv_large(const FftconvArgs&) { return hipErrorNotSupported; }

}  // namespace hyena
