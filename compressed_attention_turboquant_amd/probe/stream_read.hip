// Streaming probes: the HBM rates plain kernels reach on this part, the
// yardsticks the library's rates are compared with (reads alone for decode;
// 4:1 and 1:4 read/write mixes for quantize and dequantize).  Not part of the
// TurboQuant path; built into its own library (libtqprobe.so) for bench.py.
//
// Every thread reads 16-byte words, four loads in flight, folds them with XOR
// and stores one word at the end, so that no load can be dropped; in a
// grid-stride loop, or (the faster pattern here) a contiguous chunk per
// workgroup at a time.  The grid fills every CU with 8 workgroups of 256 threads.  With
// plain loads the same kernel also serves bench.py as a cache flush: reading
// 2 GiB of unrelated data leaves none of a workload's cache and no dirty lines
// in the 256 MB last-level cache.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// NT: non-temporal loads (no allocation in the last-level cache) or plain
// loads (which evict what the cache held, writing back dirty lines first).
template <bool NT>
__device__ __forceinline__ u4 ld(const u4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool NT>
__global__ void __launch_bounds__(256) stream_read_kernel(const u4* __restrict__ src, int64_t words,
                                                          u4* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < words; i += 4 * stride) {
    const u4 a = ld<NT>(src + i);
    const u4 b = ld<NT>(src + i + stride);
    const u4 c = ld<NT>(src + i + 2 * stride);
    const u4 d = ld<NT>(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < words; i += stride) acc ^= src[i];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Mixed streams of plain 16-byte loads and stores: each thread, per step,
// either reads four words and writes their XOR (READ4 = true: 4 bytes read per
// byte written, the shape of a quantize call, fp16 rows in and codes out) or
// reads one word and writes it to four places (1 byte read per 4 written, a
// dequantize call's shape).  `words` counts the smaller side.
template <bool READ4>
__global__ void __launch_bounds__(256) stream_rw_kernel(const u4* __restrict__ src, u4* __restrict__ dst,
                                                        int64_t words) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) {
    const int64_t base = (i / stride) * 4 * stride + i % stride;  // four words stride apart
    if constexpr (READ4) {
      dst[i] = src[base] ^ src[base + stride] ^ src[base + 2 * stride] ^ src[base + 3 * stride];
    } else {
      const u4 v = src[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[base + k * stride] = v + (uint32_t)k;
    }
  }
}

// The same streams with each workgroup taking one contiguous chunk of kChunk
// words at a time (chunks dealt to workgroups in turn), four loads in flight
// per thread, two workgroups per CU.  On this part this pattern reads about
// 15% faster than the grid-stride one above (7.1-7.2 vs 6.0-6.2 TB/s):
// requests spread over the whole buffer instead of one narrow window moving
// through it.
constexpr int64_t kChunk = 16384;  // 256 KiB per chunk

template <bool NT>
__global__ void __launch_bounds__(256) chunk_read_kernel(const u4* __restrict__ src, int64_t words,
                                                         u4* __restrict__ sink) {
  u4 acc = {0u, 0u, 0u, 0u};
  for (int64_t c0 = (int64_t)blockIdx.x * kChunk; c0 < words; c0 += (int64_t)gridDim.x * kChunk) {
    const int64_t c1 = c0 + kChunk < words ? c0 + kChunk : words;
    for (int64_t i = c0 + threadIdx.x; i < c1; i += 4 * 256) {
      u4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t j = i + 256 * k;
        v[k] = j < c1 ? ld<NT>(src + j) : u4{0u, 0u, 0u, 0u};
      }
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Chunked read/write mixes: READ4 writes dst[i] = XOR of src[4i .. 4i + 3]
// (4 bytes read per byte written), else dst[4i + k] = src[i] + k.  `words`
// counts the smaller side; chunks are kChunk words of it.
template <bool READ4>
__global__ void __launch_bounds__(256) chunk_rw_kernel(const u4* __restrict__ src, u4* __restrict__ dst,
                                                       int64_t words) {
  for (int64_t c0 = (int64_t)blockIdx.x * kChunk; c0 < words; c0 += (int64_t)gridDim.x * kChunk) {
    const int64_t c1 = c0 + kChunk < words ? c0 + kChunk : words;
    for (int64_t i = c0 + threadIdx.x; i < c1; i += 256) {
      if constexpr (READ4) {
        dst[i] = src[4 * i] ^ src[4 * i + 1] ^ src[4 * i + 2] ^ src[4 * i + 3];
      } else {
        const u4 v = src[i];
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[4 * i + k] = v + (uint32_t)k;
      }
    }
  }
}

}  // namespace

extern "C" {

// Threads the probe launches (the sink must hold this many 16-byte words).
int64_t tq_probe_stream_threads(void) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  return (int64_t)cus * 8 * 256;
}

// Reads `bytes` (a multiple of 16) at device pointer src once, with
// non-temporal loads if nontemporal != 0, else with plain loads; sink: device
// memory of tq_probe_stream_threads() * 16 bytes.  Returns a hipError_t.
int tq_probe_stream_read(const void* src, int64_t bytes, void* sink, int nontemporal, void* stream) {
  const int64_t threads = tq_probe_stream_threads();
  const dim3 grid((unsigned)(threads / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u4* s = static_cast<const u4*>(src);
  u4* k = static_cast<u4*>(sink);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, grid, dim3(256), 0, st, s, bytes / 16, k);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, grid, dim3(256), 0, st, s, bytes / 16, k);
  return (int)hipGetLastError();
}

// Mixed read/write stream: read4 != 0 reads 4 * words 16-byte words at src and
// writes words at dst; read4 == 0 reads words at src and writes 4 * words at
// dst (words a multiple of tq_probe_stream_threads()).  Returns a hipError_t.
int tq_probe_stream_rw(const void* src, void* dst, int64_t words, int read4, void* stream) {
  const int64_t threads = tq_probe_stream_threads();
  const dim3 grid((unsigned)(threads / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (words % threads) return (int)hipErrorInvalidValue;
  if (read4)
    hipLaunchKernelGGL(stream_rw_kernel<true>, grid, dim3(256), 0, st, static_cast<const u4*>(src),
                       static_cast<u4*>(dst), words);
  else
    hipLaunchKernelGGL(stream_rw_kernel<false>, grid, dim3(256), 0, st, static_cast<const u4*>(src),
                       static_cast<u4*>(dst), words);
  return (int)hipGetLastError();
}

// Workgroups of the chunked probes: two per CU.
static int64_t chunk_grid() { return tq_probe_stream_threads() / 256 / 4; }

// The chunked read: same arguments as tq_probe_stream_read.
int tq_probe_chunk_read(const void* src, int64_t bytes, void* sink, int nontemporal, void* stream) {
  const dim3 grid((unsigned)chunk_grid());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u4* s = static_cast<const u4*>(src);
  u4* k = static_cast<u4*>(sink);
  if (nontemporal)
    hipLaunchKernelGGL(chunk_read_kernel<true>, grid, dim3(256), 0, st, s, bytes / 16, k);
  else
    hipLaunchKernelGGL(chunk_read_kernel<false>, grid, dim3(256), 0, st, s, bytes / 16, k);
  return (int)hipGetLastError();
}

// The chunked read/write mixes: same arguments as tq_probe_stream_rw (any word count).
int tq_probe_chunk_rw(const void* src, void* dst, int64_t words, int read4, void* stream) {
  const dim3 grid((unsigned)chunk_grid());
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (read4)
    hipLaunchKernelGGL(chunk_rw_kernel<true>, grid, dim3(256), 0, st, static_cast<const u4*>(src),
                       static_cast<u4*>(dst), words);
  else
    hipLaunchKernelGGL(chunk_rw_kernel<false>, grid, dim3(256), 0, st, static_cast<const u4*>(src),
                       static_cast<u4*>(dst), words);
  return (int)hipGetLastError();
}

}  // extern "C"
