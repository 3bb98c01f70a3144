// Stand-ins for the kernel launchers, linked with the C ABI layer in the
// host-sanitizer build (test infrastructure).  The driver only makes calls
// that argument validation rejects, so none of these is reached; if one
// were, it would report an error instead of launching anything.
#include "../../speculative_decoding_verify_attn_amd/csrc/sv_internal.hpp"

namespace sv {
hipError_t launch_attn_mfma(const AttnParams &, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_valu(const AttnParams &, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_merge(const AttnParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sample(const SampleParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sample_tree(const SampleParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_clear(void *, size_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_tree_commit(const TreeCommitParams &, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_kv_append(const AppendParams &, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_check_inputs(const CheckParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_probe_read(const void *, size_t, float *, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_rollback(const int32_t *, int32_t *, int32_t *, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sv
