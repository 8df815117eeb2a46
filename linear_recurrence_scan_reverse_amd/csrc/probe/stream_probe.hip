// stream_probe.hip -- a measurement aid for bench.py, built as its own library
// (libstreamprobe.so) and not part of librlscan.
//
// Plain streaming kernels that move the same arrays as one estimator call: NR
// float32 inputs and NF one-byte flag arrays read, NW float32 outputs written,
// n elements each, nothing computed but a sum.  bench.py times every shape
// below on every estimator's byte mix and takes the fastest as that mix's
// practical ceiling at the call's size (launch, fill and drain included), so an
// estimator's time can be read against the best plain kernel moving its bytes,
// not only against the HBM peak.
//
// Shapes (every access non-temporal, every load instruction of a wave one
// contiguous run of 64 x 16 bytes):
//   0  grid16    one 16-byte access per lane and float array (4 flag bytes),
//                256-thread blocks, a grid that covers the data
//   1  grid32    two 16-byte accesses per lane and array (a block covers 2048
//                elements; the lane's second chunk is 4 KiB further on)
//   2  grid64    four 16-byte accesses per lane and array
//   3  grid16w   one 16-byte access per lane, 1024-thread blocks
//   4  persist   a resident grid (8 blocks of 256 threads per compute unit)
//                striding over 1024-element tiles, the next tile's loads
//                issued before the current tile's stores
//   5  grid32w   two 16-byte accesses per lane, 512-thread blocks
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kShapes = 6;

struct ProbeArgs {
  const f4* in[5];
  const uint32_t* fl[2];
  f4* out[2];
  int64_t n4;  // elements / 4
};

// U chunks of 16 bytes per lane, blocks of B threads; chunk u of lane l in
// block b covers float4 index (b * U + u) * B + l.
template <int NR, int NF, int NW, int U, int B>
__global__ void __launch_bounds__(B) grid_kernel(const ProbeArgs a) {
  const int64_t base = (int64_t)blockIdx.x * U * B + threadIdx.x;
  f4 s[U];
  uint32_t m[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    s[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    m[u] = 0;
  }
#pragma unroll
  for (int k = 0; k < NR; ++k)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * B;
      if (i < a.n4) s[u] += __builtin_nontemporal_load(a.in[k] + i);
    }
#pragma unroll
  for (int k = 0; k < NF; ++k)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * B;
      if (i < a.n4) m[u] |= __builtin_nontemporal_load(a.fl[k] + i);
    }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + u * B;
    if (m[u] & 0x01010101u) s[u].x += 1.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k)
      if (i < a.n4) __builtin_nontemporal_store(s[u] + (float)k, a.out[k] + i);
  }
}

// Resident grid striding over tiles of 256 x 4 float4 (one 16-byte access per
// lane and array for each of 4 sub-tiles); the loads of tile j + 1 are issued
// before the stores of tile j.
template <int NR, int NF, int NW>
__global__ void __launch_bounds__(256) persist_kernel(const ProbeArgs a) {
  constexpr int U = 4;
  const int64_t tiles = (a.n4 + U * 256 - 1) / (U * 256);
  f4 s[U];
  uint32_t m[U];
  auto load = [&](int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      m[u] = 0;
      const int64_t i = (t * U + u) * 256 + threadIdx.x;
      if (t < tiles && i < a.n4) {
#pragma unroll
        for (int k = 0; k < NR; ++k) s[u] += __builtin_nontemporal_load(a.in[k] + i);
#pragma unroll
        for (int k = 0; k < NF; ++k) m[u] |= __builtin_nontemporal_load(a.fl[k] + i);
      }
    }
  };
  int64_t t = blockIdx.x;
  load(t);
  for (; t < tiles; t += gridDim.x) {
    f4 cs[U];
    uint32_t cm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cs[u] = s[u];
      cm[u] = m[u];
    }
    load(t + gridDim.x);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = (t * U + u) * 256 + threadIdx.x;
      if (cm[u] & 0x01010101u) cs[u].x += 1.0f;
      if (i < a.n4) {
#pragma unroll
        for (int k = 0; k < NW; ++k) __builtin_nontemporal_store(cs[u] + (float)k, a.out[k] + i);
      }
    }
  }
}

int g_cus = 0;

template <int NR, int NF, int NW>
hipError_t launch(const ProbeArgs& a, int shape, hipStream_t st) {
  auto grid = [&](int per_block) { return dim3((unsigned)((a.n4 + per_block - 1) / per_block)); };
  switch (shape) {
    case 0: hipLaunchKernelGGL((grid_kernel<NR, NF, NW, 1, 256>), grid(256), dim3(256), 0, st, a); break;
    case 1: hipLaunchKernelGGL((grid_kernel<NR, NF, NW, 2, 256>), grid(512), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((grid_kernel<NR, NF, NW, 4, 256>), grid(1024), dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((grid_kernel<NR, NF, NW, 1, 1024>), grid(1024), dim3(1024), 0, st, a); break;
    case 4: {
      if (g_cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&g_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || g_cus <= 0)
          g_cus = 256;
      }
      const int64_t tiles = (a.n4 + 1023) / 1024;
      const int64_t want = (int64_t)g_cus * 8;
      const unsigned blocks = (unsigned)(tiles < want ? tiles : want);
      hipLaunchKernelGGL((persist_kernel<NR, NF, NW>), dim3(blocks), dim3(256), 0, st, a);
      break;
    }
    default: hipLaunchKernelGGL((grid_kernel<NR, NF, NW, 2, 512>), grid(1024), dim3(512), 0, st, a); break;
  }
  return hipGetLastError();
}

template <int NR, int NF>
hipError_t by_nw(const ProbeArgs& a, int nw, int shape, hipStream_t st) {
  return nw == 1 ? launch<NR, NF, 1>(a, shape, st) : launch<NR, NF, 2>(a, shape, st);
}

template <int NR>
hipError_t by_nf(const ProbeArgs& a, int nf, int nw, int shape, hipStream_t st) {
  switch (nf) {
    case 0: return by_nw<NR, 0>(a, nw, shape, st);
    case 1: return by_nw<NR, 1>(a, nw, shape, st);
    default: return by_nw<NR, 2>(a, nw, shape, st);
  }
}

// Checks one buffer set and fills the kernel arguments; -1 if outside the contract.
int make_args(const float* const* ins, int nr, const uint8_t* const* flags, int nf, float* const* outs, int nw,
              int64_t n, ProbeArgs& a) {
  if (!ins || !outs || nr < 1 || nr > 5 || nf < 0 || nf > 2 || nw < 1 || nw > 2 || n <= 0 || n % 4 != 0) return -1;
  if (nf > 0 && !flags) return -1;
  a = ProbeArgs{};
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
  return 0;
}

hipError_t launch_any(const ProbeArgs& a, int nr, int nf, int nw, int shape, hipStream_t st) {
  switch (nr) {
    case 1: return by_nf<1>(a, nf, nw, shape, st);
    case 2: return by_nf<2>(a, nf, nw, shape, st);
    case 3: return by_nf<3>(a, nf, nw, shape, st);
    case 4: return by_nf<4>(a, nf, nw, shape, st);
    default: return by_nf<5>(a, nf, nw, shape, st);
  }
}

}  // namespace

extern "C" {

// Number of probe shapes (valid shape arguments are 0 .. count - 1).
int stream_probe_shapes(void) { return kShapes; }

// Enqueue one probe launch of shape 0 on `stream` (kept for callers of the
// single-shape probe).  ins: nr (1..5) device pointers to float32 arrays of n
// elements; flags: nf (0..2) device pointers to n bytes; outs: nw (1..2) device
// pointers to float32 arrays of n elements (written).  n must be a positive
// multiple of 4, float arrays 16-byte aligned and flag arrays 4-byte aligned.
// Returns 0 on success, -1 for arguments outside that contract (nothing
// launched), or the hipError_t of the launch.
int stream_probe(const float* const* ins, int nr, const uint8_t* const* flags, int nf, float* const* outs, int nw,
                 int64_t n, hipStream_t stream) {
  ProbeArgs a;
  if (make_args(ins, nr, flags, nf, outs, nw, n, a) != 0) return -1;
  return (int)launch_any(a, nr, nf, nw, 0, stream);
}

// Average per-launch time (us, written to *us) of `reps` back-to-back launches
// of one shape on `stream`, launch i using buffer set i % nsets (so the sets
// can exceed the caches), timed with HIP events on that stream after one
// untimed pass over every set.  ins, flags and outs hold nsets consecutive
// groups of nr, nf and nw pointers.  Returns 0, -1 for arguments outside the
// contract of stream_probe, or a hipError_t.
int stream_probe_time(const float* const* ins, int nr, const uint8_t* const* flags, int nf, float* const* outs,
                      int nw, int64_t n, int nsets, int shape, int reps, hipStream_t stream, float* us) {
  if (nsets < 1 || nsets > 64 || reps < 1 || shape < 0 || shape >= kShapes || !us) return -1;
  ProbeArgs a[64];
  for (int i = 0; i < nsets; ++i)
    if (make_args(ins + i * nr, nr, flags ? flags + i * nf : nullptr, nf, outs + i * nw, nw, n, a[i]) != 0)
      return -1;
  hipError_t e = hipSuccess;
  for (int i = 0; i < nsets && e == hipSuccess; ++i) e = launch_any(a[i], nr, nf, nw, shape, stream);
  if (e != hipSuccess) return (int)e;
  hipEvent_t t0, t1;
  if ((e = hipEventCreate(&t0)) != hipSuccess) return (int)e;
  if ((e = hipEventCreate(&t1)) != hipSuccess) {
    (void)hipEventDestroy(t0);
    return (int)e;
  }
  e = hipEventRecord(t0, stream);
  for (int i = 0; i < reps && e == hipSuccess; ++i) e = launch_any(a[i % nsets], nr, nf, nw, shape, stream);
  if (e == hipSuccess) e = hipEventRecord(t1, stream);
  if (e == hipSuccess) e = hipEventSynchronize(t1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, t0, t1);
  (void)hipEventDestroy(t0);
  (void)hipEventDestroy(t1);
  if (e != hipSuccess) return (int)e;
  *us = ms * 1000.0f / (float)reps;
  return 0;
}

}  // extern "C"
