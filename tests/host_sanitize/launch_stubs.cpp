// Stand-ins for the HIP launchers of libringattn, for a host-only build of the
// C ABI (ringattn_abi.cpp) with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer.  No GPU code is compiled: every launcher records
// the work size it was handed and returns success without touching the
// (made-up) device pointers, so that validation, planning, the schedule and
// the layout maps run under the sanitizers with no GPU present.
#include <hip/hip_runtime.h>

#include "kernels.h"

extern "C" {
// read by the stubbed-launch tests through ctypes
int ra_hostcheck_launches = 0;     // launcher calls so far
long long ra_hostcheck_last_work = -1;  // workgroups (or rows) of the last call
int ra_hostcheck_last_xcd = -1;    // workgroup-to-XCD order of the last forward-kernel call

const char* hipGetErrorString(hipError_t) { return "stubbed HIP runtime"; }
}

namespace {
hipError_t note(long long work) {
  ++ra_hostcheck_launches;
  ra_hostcheck_last_work = work;
  return hipSuccess;
}
}  // namespace

namespace ra {
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t) {
  ra_hostcheck_last_xcd = a.xcd_swizzle;
  return note(a.n_work);
}
hipError_t launch_attn_fwd_f32(const FwdArgs& a, hipStream_t) {
  ra_hostcheck_last_xcd = a.xcd_swizzle;
  return note(a.n_work);
}
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t) { return note((long long)a.f.batch * a.f.hq * a.q_rows); }
hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, hipStream_t) { return note(a.f.n_work); }
hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs& a, hipStream_t) { return note(a.n_work_kv); }
hipError_t launch_state_init(const RowsArgs& g, float*, float*, float*, hipStream_t) {
  return note((long long)g.batch * g.heads * g.rows);
}
hipError_t launch_finalize(const RowsArgs& g, const float*, const float*, const float*, void*, int32_t, float*,
                           hipStream_t) {
  return note((long long)g.batch * g.heads * g.rows);
}
hipError_t launch_merge(const RowsArgs& g, const float*, const float*, const float*, const float*, float*, float*,
                        hipStream_t) {
  return note((long long)g.batch * g.heads * g.rows);
}
hipError_t launch_split_merge(const RowsArgs& g, int32_t, const float*, const float*, void*, int32_t, float*,
                              hipStream_t) {
  return note((long long)g.batch * g.heads * g.rows);
}
hipError_t bwd_scratch(hipStream_t, void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(1) << 30);  // made up, never dereferenced
  return hipSuccess;
}
hipError_t launch_permute(const PermuteArgs& p, int, const void*, void*, hipStream_t) {
  return note(p.batch * p.heads * p.seq);
}
}  // namespace ra
