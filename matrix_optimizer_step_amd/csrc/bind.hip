// Per-call descriptor binding: the caller's device pointers of this call are
// written into the descriptors the step's launches read (see BindMode in
// common.hpp); and table uploads through kernel arguments.  The pointers travel in the kernel's by-value arguments, so a
// call allocates nothing, copies nothing from host memory and leaves no host
// buffer that must outlive it; the descriptors land in stream order before the
// launches that read them.
#include "common.hpp"

namespace matopt {

namespace {

template <class P>
__device__ __forceinline__ P reloc(const char* base, P off) {
  return (P)(base + (uintptr_t)off);
}

__global__ __launch_bounds__(128) void bind_kernel(BindArgs a) {
  const int i = threadIdx.x;
  if (i >= a.n) return;
  const int k = a.first + i;
  const BindPtrs q = a.ptr[i];
  if (a.mode == BIND_VEC) {
    VecDesc d = ((const VecDesc*)a.tmpl)[k];
    d.p = const_cast<void*>(q.p[0]);
    d.g = q.p[1];
    d.m = (float*)q.p[2];
    d.v = (float*)q.p[3];
    ((VecDesc*)a.dst)[k] = d;
    return;
  }
  MatDesc d = ((const MatDesc*)a.tmpl)[k];
  d.w = const_cast<void*>(q.p[0]);
  d.g = q.p[1];
  d.v = const_cast<void*>(q.p[2]);
  d.o = const_cast<void*>(q.p[3]);
  if (a.mode == BIND_NS) {
    d.x[0] = reloc(a.base, d.x[0]);
    d.x[1] = reloc(a.base, d.x[1]);
    d.a = reloc(a.base, d.a);
    d.b = reloc(a.base, d.b);
    d.xs = reloc(a.base, d.xs);
    d.partials = reloc(a.base, d.partials);
    d.x0in = d.x0_is_v ? d.v : d.x[0];
  } else if (a.mode == BIND_COLCUT) {
    d.partials = reloc(a.base, d.partials);
  }
  ((MatDesc*)a.dst)[k] = d;
}

// Copies a.n bytes (a multiple of 16) from the arguments to a.dst.
__global__ __launch_bounds__(256) void upload_kernel(UploadArgs a) {
  const uint32_t i = threadIdx.x * 16u;
  if (i >= a.n) return;
  const uint4 v = *(const uint4*)(a.data + i);
  *(uint4*)((uint8_t*)a.dst + i) = v;
}

}  // namespace

hipError_t launch_upload(const UploadArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(kUploadBytes / 16), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bind(const BindArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bind_kernel, dim3(1), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace matopt
