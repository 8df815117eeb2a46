// stream_probe.hip -- a measurement aid for bench.py, built as its own library
// (libstreamprobe.so) and not part of librlscan.
//
// The plain streaming kernel that moves the same arrays as one estimator call:
// NR float32 inputs and NF one-byte flag arrays read, NW float32 outputs
// written, n elements each, nothing computed but a sum.  bench.py times it next
// to each estimator, so an estimator's time can be read against the best a
// kernel of that byte mix does at that size (launch fill and drain included),
// not only against the HBM peak.
//
// Shape: one 16-byte non-temporal access per lane per float array (4 bytes per
// flag array), a grid that covers the data, blocks of 256 threads.  Measured on
// one MI355X this was the fastest of the plain shapes tried: grid-stride loops
// over a resident grid ran 3-8% slower, temporal accesses 5-15% slower.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

struct ProbeArgs {
  const f4* in[5];
  const uint32_t* fl[2];
  f4* out[2];
  int64_t n4;  // elements / 4
};

template <int NR, int NF, int NW>
__global__ void __launch_bounds__(256) probe_kernel(const ProbeArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n4) return;
  f4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < NR; ++k) s += __builtin_nontemporal_load(a.in[k] + i);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < NF; ++k) m |= __builtin_nontemporal_load(a.fl[k] + i);
  if (m & 0x01010101u) s.x += 1.0f;
#pragma unroll
  for (int k = 0; k < NW; ++k) __builtin_nontemporal_store(s + (float)k, a.out[k] + i);
}

template <int NR, int NF, int NW>
hipError_t launch(const ProbeArgs& a, hipStream_t st) {
  const unsigned blocks = (unsigned)((a.n4 + 255) / 256);
  hipLaunchKernelGGL((probe_kernel<NR, NF, NW>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int NR, int NF>
hipError_t by_nw(const ProbeArgs& a, int nw, hipStream_t st) {
  return nw == 1 ? launch<NR, NF, 1>(a, st) : launch<NR, NF, 2>(a, st);
}

template <int NR>
hipError_t by_nf(const ProbeArgs& a, int nf, int nw, hipStream_t st) {
  switch (nf) {
    case 0: return by_nw<NR, 0>(a, nw, st);
    case 1: return by_nw<NR, 1>(a, nw, st);
    default: return by_nw<NR, 2>(a, nw, st);
  }
}

}  // namespace

// Enqueue one probe launch on `stream`.  ins: nr (1..5) device pointers to
// float32 arrays of n elements; flags: nf (0..2) device pointers to n bytes;
// outs: nw (1..2) device pointers to float32 arrays of n elements (written).
// n must be a positive multiple of 4, float arrays 16-byte aligned and flag
// arrays 4-byte aligned.  Returns 0 on success, -1 for arguments outside that
// contract (nothing launched), or the hipError_t of the launch.
extern "C" int stream_probe(const float* const* ins, int nr, const uint8_t* const* flags, int nf,
                            float* const* outs, int nw, int64_t n, hipStream_t stream) {
  if (!ins || !outs || nr < 1 || nr > 5 || nf < 0 || nf > 2 || nw < 1 || nw > 2 || n <= 0 || n % 4 != 0)
    return -1;
  if (nf > 0 && !flags) return -1;
  ProbeArgs a{};
  for (int k = 0; k < nr; ++k) {
    if (!ins[k] || (uintptr_t)ins[k] % 16 != 0) return -1;
    a.in[k] = reinterpret_cast<const f4*>(ins[k]);
  }
  for (int k = 0; k < nf; ++k) {
    if (!flags[k] || (uintptr_t)flags[k] % 4 != 0) return -1;
    a.fl[k] = reinterpret_cast<const uint32_t*>(flags[k]);
  }
  for (int k = 0; k < nw; ++k) {
    if (!outs[k] || (uintptr_t)outs[k] % 16 != 0) return -1;
    a.out[k] = reinterpret_cast<f4*>(outs[k]);
  }
  a.n4 = n / 4;
  hipError_t e;
  switch (nr) {
    case 1: e = by_nf<1>(a, nf, nw, stream); break;
    case 2: e = by_nf<2>(a, nf, nw, stream); break;
    case 3: e = by_nf<3>(a, nf, nw, stream); break;
    case 4: e = by_nf<4>(a, nf, nw, stream); break;
    default: e = by_nf<5>(a, nf, nw, stream); break;
  }
  return (int)e;
}
