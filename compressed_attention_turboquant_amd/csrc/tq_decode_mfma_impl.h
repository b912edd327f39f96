#pragma once
// Decode attention on the compressed cache with the matrix cores (gfx950):
// the split kernel and its device helpers.  Included by tq_decode_mfma_inst.hip,
// which the build compiles once per head dimension and key kind, so that the
// instantiations compile in parallel.
//
// What is computed is the asymmetric estimator and softmax of [cuTile]
// listing (asymmetric score estimator; fused attention function with online
// softmax and values decoded on chip), with the query
// rotated once ([Mobilint] "Two-Stage Approach": <q, x~> = <Pi q, y~>):
//   s_t = n_t * (<R q, c_k[idx_t]> + gamma_t sqrt(pi/2)/d <S q, sigma_t>) / sqrt(d)
//   out = R^T (sum_t softmax(s)_t * nv_t * c_v[idxv_t]).
//
// How it maps to CDNA4 (one 64-lane wave works on 32 keys at a time):
//  * Set-up per workgroup: the first key blocks start loading; the code tables
//    are filled; the workgroup's query rows are rotated once (R q, S q in fp32)
//    and normalised for the fp16 operand split.
//  * Both contractions run on v_mfma_f32_16x16x32_f16.  Scores: with row groups
//    of 4 the 16 MFMA rows are 4 query rows x {R q hi, R q lo, S q hi, S q lo}
//    (the centroid term's A operand fills the first two parts, the sign term's
//    the other two); with row groups of 8 (heads with more than 4 query rows)
//    they are 8 query rows x {hi, lo} in both operands.  The B operands are the
//    decoded centroids and the sign values of 16 keys.  P.V: rows are {p hi,
//    p lo} per query row against the decoded value centroids; the sum stays in
//    the rotated domain.
//  * The fp32 query splits into hi + lo halves (exact to ~2^-22).  Centroids are
//    used as fp16 copies of s*c with a per-codebook factor s chosen at set-up so
//    every s*c_i is within 2e-5 (3-bit) / 1e-4 (4-bit) of an fp16 value; 1/s is
//    folded into the query side.
//  * Code -> fp16 decode is a table lookup in LDS: for widths 1-3 the packed
//    stream's next four codes form the index of an 8-byte entry holding their
//    four fp16 values (4-bit codes: pairs, 4-byte entries).  Two VALU ops (an
//    align and a mask) and one 64-bit LDS read per four codes; the workgroup
//    fills the table (32 KB for 3-bit codes) once at start.
//  * Sign bits become fp16 B-operand halves by masking: a half whose only set
//    bit is exponent bit p is the power of two 2^(2^(p-10)-15); rotating the
//    32 sign bits by 0/4/8/12 and masking bits p and p+16 (p = 10..13) yields
//    16 dwords with one AND each.  The query side carries the matching 2^(15 -
//    2^(p-10)) factors, so the MFMA returns sum_{sigma=+1} S q and the sign term
//    is 2 * that - sum S q.
//  * Softmax runs in the log2 domain with a lazily updated running maximum: the
//    accumulators are rescaled only in the (rare) blocks where a score exceeds
//    the current maximum of its row.
//  * Split-K over keys: grid (sequence x row group, split), sized so the
//    workgroups fill the chip once; 4 waves per workgroup take every 4th block
//    of 32 keys, each keeping two blocks of loads in flight (three rotating
//    register sets; d = 256 keeps two sets and decodes in smaller pieces so that
//    two waves fit per SIMD); the waves' partial (max, sum, acc) merge in LDS
//    and one partial per split goes to the workspace; a small kernel merges the
//    splits and un-rotates.  (Merging in the last workgroup instead needs an
//    agent-scope fence per workgroup, which writes back the L2 of its XCD and
//    cost more than the extra launch.)
//  * Loads go through buffer descriptors with per-sequence SGPR bases: 32-bit
//    offsets, and reads past the capacity (or past N for the norms) return 0.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>
#include <type_traits>

#include "tq_kernels.h"
#include "tq_lanes.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kSlack = 4.f;            // log2 headroom of the lazily updated maximum
constexpr float kInvSlack = 1.f / 16.f;  // 2^-kSlack
// The P.V operand p * ||v|| * vsc is kept below 2^15 (fp16 holds up to 65504):
// with p <= 2^kSlack that needs ||v|| * vsc <= 2^kVExp.
constexpr int kVExp = 11;

template <int I, int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor<I + 1, N>(f);
  }
}

// Code -> fp16 operand tables in LDS.  Widths 1-3 look codes up four at a time:
// a 4*BITS-bit index selects an 8-byte entry holding the four fp16 centroids, one
// 64-bit LDS read per four codes.  4-bit codes go in pairs: an 8-bit index
// selects a 4-byte entry of two fp16 centroids.  (A random 64-bit read from such
// a table costs about as much LDS time as a 32-bit cross-lane permute, so four
// codes per read halve the LDS time of two codes per permute.)
template <int BITS>
struct Lut {
  static constexpr int kCodes = BITS < 4 ? 4 : 2;   // codes per lookup
  static constexpr int kIdx = BITS * kCodes;        // index bits
  static constexpr int kEntries = 1 << kIdx;
  static constexpr int kShift = kCodes == 4 ? 3 : 2;  // log2 of the entry bytes
  static constexpr int kDwords = kEntries << (kShift - 2);
};

// Bits [O, O+N) of the little-endian stream in w[], moved to bits [SH, SH+N) of
// the result, every other bit zero: a byte offset into a table of 2^SH-byte
// entries.
template <int O, int N, int SH, int NW>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[NW]) {
  constexpr uint32_t mask = ((1u << N) - 1u) << SH;
  constexpr int b = O - SH;
  if constexpr (b < 0) {
    return (w[0] << (-b)) & mask;
  } else {
    constexpr int wi = b / 32, sh = b % 32;
    static_assert(wi < NW && (wi + 1 < NW || sh + SH + N <= 32), "field outside the stream");
    if constexpr (sh == 0)
      return w[wi] & mask;
    else if constexpr (wi + 1 < NW)
      return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
    else
      return (w[wi] >> sh) & mask;
  }
}

// The eight fp16 centroids (s * c[code]) of the codes at stream bit offsets
// O, O+BITS, ..., O+7*BITS, in order, as one MFMA operand.
template <int BITS, int O, int NW>
__device__ __forceinline__ u4 decode8(const uint32_t (&w)[NW], const uint32_t* tab) {
  using L = Lut<BITS>;
  const char* base = reinterpret_cast<const char*>(tab);
  u4 r;
  if constexpr (L::kCodes == 4) {
    const u2 lo = *reinterpret_cast<const u2*>(base + field<O, L::kIdx, 3>(w));
    const u2 hi = *reinterpret_cast<const u2*>(base + field<O + 4 * BITS, L::kIdx, 3>(w));
    r[0] = lo[0];
    r[1] = lo[1];
    r[2] = hi[0];
    r[3] = hi[1];
  } else {
    sfor<0, 4>([&](auto i) {
      r[decltype(i)::value] = *reinterpret_cast<const uint32_t*>(base + field<O + 8 * decltype(i)::value, 8, 2>(w));
    });
  }
  return r;
}

__device__ __forceinline__ uint32_t half_bits(float x) {
  return (uint32_t)__half_as_ushort(__float2half_rn(x));
}

// Every thread of the workgroup: fill the table for centroids c scaled by s.
// Lane l holds the fp16 pair of the codes in the low and high half of its lane
// index (one code per half for 4-bit tables).  A wave fills 64 consecutive
// entries, so an entry's low half is the lane's own value and its high half
// comes from the lane its high index bits name (one cross-lane read).
template <int BITS, int T>
__device__ __forceinline__ void fill_lut(uint32_t* tab, const float* c, float s, int tid) {
  using L = Lut<BITS>;
  constexpr uint32_t m = (1u << BITS) - 1u;
  const int lane = tid % 64;
  if constexpr (L::kCodes == 4) {
    constexpr int pb = 2 * BITS;  // bits of a pair index; 2^pb divides 64
    constexpr uint32_t pm = (1u << pb) - 1u;
    const uint32_t P = half_bits(s * c[lane & m]) | (half_bits(s * c[(lane >> BITS) & m]) << 16);
    for (int i0 = 0; i0 < L::kEntries; i0 += T) {
      const uint32_t i = (uint32_t)(i0 + tid);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((i >> pb) & pm) << 2), (int)P);
      if (i < (uint32_t)L::kEntries) *reinterpret_cast<u2*>(tab + 2 * i) = u2{P, hi};
    }
  } else {
    const uint32_t h = half_bits(s * c[lane & m]);
    for (int i0 = 0; i0 < L::kEntries; i0 += T) {
      const uint32_t i = (uint32_t)(i0 + tid);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((i >> BITS) & m) << 2), (int)h);
      if (i < (uint32_t)L::kEntries) tab[i] = h | (hi << 16);
    }
  }
}

// Column tables for 4-bit codes: 32 copies of the 256-entry pair table (two
// fp16 centroids per 4-byte entry), entry e of copy c at dword e * 32 + c.
// Lane l reads copy l % 32, so every lane of a 32-lane half reads its own bank
// whatever the codes (random entries of one shared 1 KB table collide in most
// reads).  32 KB.
constexpr int kColDwords4 = 256 * 32;

template <int T>
__device__ __forceinline__ void fill_lut_cols4(uint32_t* tab, const float* c, float s, int tid) {
  for (int i = tid; i < 256 * 32; i += T) {
    const int e = i / 32;
    tab[i] = half_bits(s * c[e & 15]) | (half_bits(s * c[e >> 4]) << 16);
  }
}

// decode8 for 4-bit codes from a column table; colp = the lane's copy (tab +
// l % 32).
template <int O, int NW>
__device__ __forceinline__ u4 decode8_cols4(const uint32_t (&w)[NW], const uint32_t* colp) {
  u4 r;
  sfor<0, 4>([&](auto i) {
    r[decltype(i)::value] = colp[32 * field<O + 8 * decltype(i)::value, 8, 0>(w)];
  });
  return r;
}

// Code -> fp16 operand lookup from the kernel's table for BITS-bit codes: the
// column table (COL, 4-bit codes) or the shared table.
template <int BITS, bool COL, int O, int NW>
__device__ __forceinline__ u4 lookup8(const uint32_t (&w)[NW], const uint32_t* tab, const uint32_t* colp) {
  if constexpr (COL)
    return decode8_cols4<O>(w, colp);
  else
    return decode8<BITS, O>(w, tab);
}

// Which tables of a (KB, VB) kernel are column tables: 4-bit ones, unless the
// other width is 3 (its 32 KB table next to a 32 KB column table would leave
// room for only one workgroup per CU).
template <int KB, int VB>
struct Tables {
  static constexpr bool kColK = KB == 4 && VB != 3, kColV = VB == 4 && KB != 3;
  static constexpr int kK = kColK ? kColDwords4 : Lut<KB>::kDwords;
  static constexpr int kV = KB == VB ? 0 : (kColV ? kColDwords4 : Lut<VB>::kDwords);
};

// Sign-term B operand: k-block kb, dword w selects exponent bit p = 10 + w of the
// sign word rotated left by 4*(kb % 4), in both halves.
template <int W>
__device__ __forceinline__ uint32_t sign_dword(uint32_t rotated) {
  return rotated & ((1u << (10 + W)) | (1u << (26 + W)));
}

// Coordinate offset (within the lane's 32 sign bits) and query-side factor of
// sign slot (kb % 4 = r, dword w, half h).
__device__ __forceinline__ int sign_coord(int r, int w, int h) {
  return (10 + w + 16 * h - 4 * r) & 31;
}
__device__ __forceinline__ float sign_comp(int w) {  // 2^(15 - 2^w)
  return w == 0 ? 16384.f : w == 1 ? 8192.f : w == 2 ? 2048.f : 128.f;
}

template <int D, int KB, int QJL, int VB>
struct Shape {
  static constexpr int KBLK = D / 32;         // k-blocks of 32 coordinates
  static constexpr int NWK = KB * D / 128;    // key-code dwords per lane per 16 keys
  static constexpr int NSW = D / 128;         // sign dwords per lane per 16 keys
  static constexpr int NWV = D * VB / 64;     // value-code dwords per lane per 32 keys
  static constexpr int CB = D / 16;           // 16-coordinate output blocks
  static constexpr int KROW = D * KB / 8;     // key-code bytes per token
  static constexpr int VTILE = D * VB;        // value-code bytes per 8-token tile
};

// Registers of one 32-key block, as this lane needs them.
template <int D, int KB, int QJL, int VB>
struct Block {
  using S = Shape<D, KB, QJL, VB>;
  uint32_t kw[2][S::NWK];
  uint32_t sw[2][QJL ? S::NSW : 1];
  float kn[2], kg[2], vn[2];
  uint32_t vw[S::NWV];
};

// Per-sequence buffer descriptors: 32-bit offsets from an SGPR base; reads past
// the described range return 0 (keys at or beyond the capacity, norms of keys
// at or beyond N).
struct SeqBuffers {
  __amdgpu_buffer_rsrc_t kidx, ksign, knorm, krnorm, vidx, vnorm;
};

constexpr int kBufCfg = 0x00020000;  // raw (untyped) buffer on gfx9
// Cache policy of the packed-cache loads (the aux operand of the buffer
// loads): kLoadNT marks them non-temporal (streamed past the caches).  In the
// split kernel the key codes, signs and norms load that way (measured in one
// run: C3 357 -> 340 us, C5 786 -> 771 us); the value tiles do not: their
// lanes read 48- or 64-byte pieces in several 16-byte loads, which then fetch
// their lines again (C5 786 -> 953 us with them non-temporal).  The
// many-rows kernel keeps the default: its row groups meet each key block in L2.
constexpr int kLoadNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufCfg);
}

template <int N, int kLoadAux = 0>
__device__ __forceinline__ void buf_load(uint32_t (&dst)[N], __amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (N == 1) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadAux);
  } else if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadAux);
    dst[0] = v[0];
    dst[1] = v[1];
  } else if constexpr (N == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, kLoadAux);
    dst[0] = v[0];
    dst[1] = v[1];
    dst[2] = v[2];
  } else {
    static_assert(N % 4 == 0 || N == 6 || N == 12, "unsupported width");
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, kLoadAux);
        dst[i] = v[0];
        dst[i + 1] = v[1];
        dst[i + 2] = v[2];
        dst[i + 3] = v[3];
      }
    } else {  // 6 or 12 dwords: b128 + b64 pieces
#pragma unroll
      for (int i = 0; i < N; i += 6) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, kLoadAux);
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * i + 16, 0, kLoadAux);
        dst[i] = v[0];
        dst[i + 1] = v[1];
        dst[i + 2] = v[2];
        dst[i + 3] = v[3];
        dst[i + 4] = u[0];
        dst[i + 5] = u[1];
      }
    }
  }
}

template <int kLoadAux = 0>
__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadAux));
}

template <int D, int KB, int QJL, int VB>
__device__ __forceinline__ void load_block(Block<D, KB, QJL, VB>& b, const SeqBuffers& sb, int k0,
                                           int l16, int g4) {
  using S = Shape<D, KB, QJL, VB>;
  constexpr int A = kLoadNT, AV = 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = k0 + 16 * t + l16;
    buf_load<S::NWK, A>(b.kw[t], sb.kidx, key * S::KROW + g4 * (S::KROW / 4));
    if constexpr (QJL) buf_load<S::NSW, A>(b.sw[t], sb.ksign, key * (D / 8) + g4 * (D / 32));
    b.kn[t] = buf_f32<A>(sb.knorm, key * 4);
    if constexpr (QJL) b.kg[t] = buf_f32<A>(sb.krnorm, key * 4);
    b.vn[t] = buf_f32<A>(sb.vnorm, key * 4);
  }
  // The tile index is below 2^24 (buffer offsets are 32-bit), so a 24-bit
  // multiply is exact; a 32-bit one compiles to a 64-bit multiply-add whose
  // unused high operand can make the loop wait for every load in flight.
  buf_load<S::NWV, AV>(b.vw, sb.vidx, (int)__umul24((unsigned)(k0 / 8 + g4), (unsigned)S::VTILE) + l16 * (S::VTILE / 16));
}

// Per-wave state of the running softmax and the query operands.  A lane holds
// NR query rows (NR = 1: the 16 MFMA rows are 4 query rows x {R q hi, R q lo,
// S q hi, S q lo}; NR = 2: they are 8 query rows x {hi, lo}, the centroid and
// sign terms having separate A operands).
template <int D, int KB, int QJL, int VB, int NR>
struct WaveState {
  using S = Shape<D, KB, QJL, VB>;
  h8 Ak[S::KBLK], As[QJL ? S::KBLK : 1];
  f4 acc[S::CB];
  float m[NR], msafe[NR], lsum[NR];
  float vsc, vlim;  // value-norm factor of the P operand (a power of two) and 2^kVExp / vsc
  float ca[NR], c2[NR], c0[NR];
  int limit[NR];
  int64_t srow[NR];
  const uint32_t *ktab, *vtab;  // code -> fp16 tables in LDS
  const uint32_t *kcol, *vcol;  // this lane's copy in a column table
  // Dithered variant: cd = sum_j (R q)_j log2(e) / sqrt(d) per row (the score
  // term of the key offset is n delta cd); dacc = sum over this lane's keys of
  // p n_v delta_v (the value offset's share, the same for every coordinate).
  float cd[NR], dacc[NR];
  float dkw, dvw;  // offset widths
  int64_t seq;
};

template <int D, int KB, int QJL, int VB, int SCORES, int NR, int DITHER>
__device__ __forceinline__ void process_block(WaveState<D, KB, QJL, VB, NR>& ws, const Block<D, KB, QJL, VB>& cur,
                                              int k0, const DecodeMfmaParams& p, _Float16 (*pb)[4 * NR][32],
                                              int l16, int g4, int rows) {
  using S = Shape<D, KB, QJL, VB>;
  // At d = 256 the decoded operands of a whole block would not fit next to two
  // waves' worth of other state, so keys are decoded one 16-key tile at a time
  // and values in two halves (kLean); the second wave on the SIMD covers the
  // LDS latency this exposes.
  constexpr bool kLean = D == 256;
  constexpr int kVParts = kLean ? 2 : 1, kCBp = S::CB / kVParts;
  f4 sk[2], ss[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sk[t] = f4{0.f, 0.f, 0.f, 0.f};
    ss[t] = sk[t];
  }
  // Score MFMAs of tile t from its decoded keys.  Separate accumulators for the
  // centroid and sign parts halve the dependency chains (with NR = 1 each fills
  // only its own rows, parts 0,1 / 2,3).
  auto score_tile = [&](int t, const u4 (&bkt)[S::KBLK]) {
    sfor<0, S::KBLK>([&](auto kb) {
      sk[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ws.Ak[kb], __builtin_bit_cast(h8, bkt[kb]), sk[t], 0, 0, 0);
      if constexpr (QJL) {
        constexpr int r = kb % 4;
        const uint32_t word = cur.sw[t][kb / 4];
        const uint32_t rot = r == 0 ? word : __builtin_amdgcn_alignbit(word, word, 32 - 4 * r);
        u4 bw;
        sfor<0, 4>([&](auto w) { bw[decltype(w)::value] = sign_dword<decltype(w)::value>(rot); });
        ss[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ws.As[kb], __builtin_bit_cast(h8, bw), ss[t], 0, 0, 0);
      }
    });
  };
  if constexpr (!kLean) {
    // Phase 1: all key-code lookups of both 16-key tiles go out before any MFMA
    // needs one, so the LDS latency overlaps instead of serialising.
    u4 bk[2][S::KBLK];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      sfor<0, S::KBLK>([&](auto kb) {
        bk[t][kb] = lookup8<KB, Tables<KB, VB>::kColK, 8 * KB * kb>(cur.kw[t], ws.ktab, ws.kcol);
      });
    __builtin_amdgcn_sched_barrier(0);
    // Phase 2: score MFMAs.
    score_tile(0, bk[0]);
    score_tile(1, bk[1]);
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u4 bk[S::KBLK];
      sfor<0, S::KBLK>([&](auto kb) {
        bk[kb] = lookup8<KB, Tables<KB, VB>::kColK, 8 * KB * kb>(cur.kw[t], ws.ktab, ws.kcol);
      });
      __builtin_amdgcn_sched_barrier(0);
      score_tile(t, bk);
    }
  }
  // Phase 3: value-code lookups (the first part at d = 256), in flight while the
  // softmax arithmetic runs.
  u4 bv[kCBp];
  sfor<0, kCBp>([&](auto cb) {
    bv[cb] = lookup8<VB, Tables<KB, VB>::kColV, 8 * VB * cb>(cur.vw, ws.vtab, ws.vcol);
  });
  __builtin_amdgcn_sched_barrier(0);
  // Dithered variant: the offsets of this lane's two keys (key and value streams).
  float dk[2] = {0.f, 0.f}, dv[2] = {0.f, 0.f};
  if constexpr (DITHER) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = k0 + 16 * t + l16;
      dk[t] = cur.kn[t] * dither_offset(p.kd0, ws.seq, key, ws.dkw);
      dv[t] = cur.vn[t] * dither_offset(p.vd0, ws.seq, key, ws.dvw);
    }
  }
  // Phase 4: scores of lane (query rows NR g4 + j, key l16), online softmax.
  float st[NR][2];
#pragma unroll
  for (int j = 0; j < NR; ++j)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float cent = NR == 1 ? sk[t][0] + sk[t][1] : sk[t][2 * j] + sk[t][2 * j + 1];
      float s = (cur.kn[t] * ws.ca[j]) * cent;
      if constexpr (DITHER) s = fmaf(dk[t], ws.cd[j], s);
      if constexpr (QJL) {
        const float sgn = NR == 1 ? ss[t][2] + ss[t][3] : ss[t][2 * j] + ss[t][2 * j + 1];
        s = fmaf(cur.kn[t] * cur.kg[t], fmaf(ws.c2[j], sgn, ws.c0[j]), s);
      }
      const int key = k0 + 16 * t + l16;
      s = key < ws.limit[j] ? s : -INFINITY;
      if constexpr (SCORES) {
        if (NR * g4 + j < rows && key < p.N) p.scores[ws.srow[j] * p.N + key] = s * kLn2;
      }
      st[j][t] = s;
    }
  // The reference maximum only moves when a score exceeds it by more than
  // kSlack (log2 units): weights stay <= 2^kSlack, and the rare rescale keeps
  // the sum exact (every term is relative to the same reference).
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const float mx = fmaxf(st[j][0], st[j][1]);
    if (__any(mx > ws.m[j] + kSlack)) {
      float rmax = mx;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o));
      const float mnew = fmaxf(ws.m[j], rmax);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(ws.m[j] - mnew);
      ws.lsum[j] *= alpha;
      if constexpr (DITHER) ws.dacc[j] *= alpha;
#pragma unroll
      for (int i = 0; i < S::CB; ++i) {
        if constexpr (NR == 1) {
          ws.acc[i] *= alpha;
        } else {
          ws.acc[i][2 * j] *= alpha;
          ws.acc[i][2 * j + 1] *= alpha;
        }
      }
      ws.m[j] = mnew;
      ws.msafe[j] = mnew == -INFINITY ? 0.f : mnew;
    }
  }
  // The value norms enter the fp16 P operand scaled by vsc.  It starts at
  // 2^-kSlack; a block whose largest norm exceeds vlim lowers it to the power of
  // two that brings that norm below 2^kVExp, and the accumulators are scaled by
  // the same exact factor (every term of the sum keeps one common scale).  The
  // block maximum is the same in every 16-lane group (they hold the same keys).
  {
    const float vl = fmaxf(cur.vn[0], cur.vn[1]);
    if (__any(vl > ws.vlim)) {
      float vm = vl;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) vm = fmaxf(vm, __shfl_xor(vm, o));
      int e = 0;
      frexpf(vm, &e);  // vm < 2^e
      const float nsc = fminf(ws.vsc, ldexpf(1.f, kVExp - e));
      const float ratio = nsc / ws.vsc;
#pragma unroll
      for (int i = 0; i < S::CB; ++i) ws.acc[i] *= ratio;
      ws.vsc = nsc;
      ws.vlim = ldexpf(1.f, kVExp) / nsc;
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    // v_exp_f32 directly: weights below 2^-126 of the running maximum become 0.
    const float p0 = __builtin_amdgcn_exp2f(st[j][0] - ws.msafe[j]);
    const float p1 = __builtin_amdgcn_exp2f(st[j][1] - ws.msafe[j]);
    ws.lsum[j] += p0 + p1;
    if constexpr (DITHER) ws.dacc[j] = fmaf(p0, dv[0], fmaf(p1, dv[1], ws.dacc[j]));
    const float q0 = p0 * cur.vn[0] * ws.vsc, q1 = p1 * cur.vn[1] * ws.vsc;
    const _Float16 h0 = (_Float16)q0, h1 = (_Float16)q1;
    const int qr = NR * g4 + j;
    pb[0][qr][l16] = h0;
    pb[0][qr][16 + l16] = h1;
    pb[1][qr][l16] = (_Float16)(q0 - (float)h0);
    pb[1][qr][16 + l16] = (_Float16)(q1 - (float)h1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  h8 ap = h8{0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (NR == 1) {
    const int part = l16 % 4, qr = l16 / 4;
    if (part < 2) ap = *reinterpret_cast<const h8*>(&pb[part][qr][8 * g4]);
  } else {
    ap = *reinterpret_cast<const h8*>(&pb[l16 % 2][l16 / 2][8 * g4]);
  }
  // Phase 5: P.V (at d = 256 the second half of the values is decoded after
  // the first half's MFMAs are issued).
  sfor<0, kCBp>([&](auto cb) {
    ws.acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(h8, bv[cb]), ws.acc[cb], 0, 0, 0);
  });
  if constexpr (kLean) {
    sfor<0, kCBp>([&](auto cb) {
      bv[cb] = lookup8<VB, Tables<KB, VB>::kColV, 8 * VB * (cb + kCBp)>(cur.vw, ws.vtab, ws.vcol);
    });
    sfor<0, kCBp>([&](auto cb) {
      ws.acc[cb + kCBp] =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(ap, __builtin_bit_cast(h8, bv[cb]), ws.acc[cb + kCBp], 0, 0, 0);
    });
  }
  __builtin_amdgcn_wave_barrier();
}

// Four of the workgroup's query rows (rb..rb+3) rotated once: rq[0][r][j] =
// (R q_r)_j / s_k and rq[1][r][j] = (S q_r)_j, from the rows in qs (LDS) and
// R^T, S^T (global, row-major).  Thread (matrix, jq, slice) reads float4 rows
// M[k][4jq..4jq+3] over its slice of k for the four rows; the slices' partial
// sums meet in part (LDS).  Each workgroup starts its slices at its own row
// offset k0, so that the workgroups, which all read the same few hundred KB at
// once, spread over the L2 channels.
template <int D, int QJL, int RW, int T>
__device__ __forceinline__ void rotate_rows(const float* __restrict__ Rt, const float* __restrict__ St,
                                            float s_k, const float (*qs)[D], float (*rq)[RW][D],
                                            f4 (*part)[4][D / 4], int tid, int k0, int rb) {
  constexpr int kJ = D / 4;                   // float4 columns per matrix row
  constexpr int kMats = D == 128 ? 2 : 1;     // matrices handled side by side
  constexpr int kSl = T / (kJ * kMats);       // k-slices: 4 per 256 threads
  constexpr int kSpan = D / kSl;
#pragma unroll
  for (int pass = 0; pass < 2 / kMats; ++pass) {
    const int m = kMats == 2 ? tid / (kJ * kSl) : pass;
    const int jq = tid % kJ, sl = (tid / kJ) % kSl;
    if (QJL || m == 0) {
      const f4* M = reinterpret_cast<const f4*>(m == 0 ? Rt : St) + jq;
      f4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
#pragma unroll 16
      for (int kk = 0; kk < kSpan; ++kk) {
        const int k = (sl * kSpan + kk + k0) & (D - 1);
        const f4 x = M[(size_t)k * kJ];
        a0 += x * qs[rb][k];
        a1 += x * qs[rb + 1][k];
        a2 += x * qs[rb + 2][k];
        a3 += x * qs[rb + 3][k];
      }
      const int ps = (kMats == 2 ? m * kSl : 0) + sl;
      part[ps][0][jq] = a0;
      part[ps][1][jq] = a1;
      part[ps][2][jq] = a2;
      part[ps][3][jq] = a3;
    }
    // part holds one matrix per pass at d = 256; at d = 128 the two matrices
    // use its two halves (slices 0-3 for R, 4-7 for S).
    __syncthreads();
    for (int o = tid; o < kMats * 4 * D; o += T) {
      const int mm = kMats == 2 ? o / (4 * D) : pass, r = (o / D) % 4, j = o % D;
      float v = 0.f;
      if (QJL || mm == 0) {
#pragma unroll
        for (int t = 0; t < kSl; ++t) v += part[(kMats == 2 ? mm * kSl : 0) + t][r][j / 4][j % 4];
      }
      rq[mm][rb + r][j] = mm == 0 ? v / s_k : v;
    }
    if (pass + 1 < 2 / kMats) __syncthreads();
  }
}

// Key blocks [b0, b1) of split `split` of this workgroup's row group.  Blocks
// are dispatched in linear order (x fastest), so with two workgroups per CU
// the first first_wgs of them share no CU and each CU's second workgroup
// arrives later; the later one runs its key loop about 11% slower (the SIMDs'
// issue arbitration favours the older waves) and, with equal splits, runs alone
// at the end while the first has finished.  Giving the first-dispatched splits
// (those with x + gx y < first_wgs, the lowest y of each row group) first_share
// / 1024 times the blocks of the others makes both end together.  The layout
// depends only on the grid, so the results do not depend on timing; a split can
// come out empty (b0 >= b1), which the merge and the combine treat as weight 0.
__device__ __forceinline__ void split_blocks(const DecodeMfmaParams& p, int split, int& b0, int& b1) {
  const int nblk = (int)((p.N + 31) / 32), ns = (int)gridDim.y, per = (int)(p.keys_per_split / 32);
  const int x = (int)blockIdx.x, gx = (int)gridDim.x;
  int nf = x < p.first_wgs ? (p.first_wgs - x + gx - 1) / gx : 0;
  nf = min(nf, ns);
  if (nf > 0 && nf < ns) {
    const int64_t S = p.first_share;
    const int big = (int)(((int64_t)nblk * S + nf * S + (int64_t)(ns - nf) * 1024 - 1) / (nf * S + (int64_t)(ns - nf) * 1024));
    const int rest = nblk - nf * big;
    const int small = (rest + ns - nf - 1) / (ns - nf);
    if (rest > 0 && small > 0) {
      b0 = split < nf ? split * big : nf * big + (split - nf) * small;
      b1 = min(nblk, b0 + (split < nf ? big : small));
      return;
    }
  }
  b0 = split * per;
  b1 = min(nblk, b0 + per);
}

// W waves per workgroup; the SIMDs hold two waves each where
// decode_simd_waves allows (the bound keeps a code change from silently
// halving occupancy).
// DITHER: the dithered variant (keys without QJL): reconstructions c[idx] + delta.
template <int D, int KB, int QJL, int VB, int SCORES, int NR, int W, int DITHER>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(decode_simd_waves(D, QJL, 4 * NR))))
decode_mfma_kernel(DecodeMfmaParams p) {
  using S = Shape<D, KB, QJL, VB>;
  constexpr int T = 64 * W;   // threads
  constexpr int RW = 4 * NR;  // query rows per workgroup
  // One table serves keys and values when their widths match (the codebook and
  // its fp16 factor depend only on the width and the head dimension).
  using TB = Tables<KB, VB>;
  __shared__ __align__(16) uint32_t lut[TB::kK + TB::kV];
  __shared__ __align__(16) _Float16 pbuf[W][2][RW][32];
  __shared__ float mrg_m[W][RW], mrg_l[W][RW];
  __shared__ float qsh[RW][D];     // the workgroup's query rows
  __shared__ float qrs[2][RW][D];  // R q / s_k and S q of those rows
  __shared__ float qcon[RW][4];    // per row: c1, c2, -sum(S q), sum(R q) (dithered variant)
  // The rotation's k-slice partial sums (set-up) and the waves' accumulators
  // (merge, after the key loop) share one buffer.
  constexpr int kRpart = (T / (D / 4)) * 4 * (D / 4) * 16, kMrg = W * RW * D * 4;
  __shared__ __align__(16) char scratch[kRpart > kMrg ? kRpart : kMrg];
  auto rpart = reinterpret_cast<f4 (*)[4][D / 4]>(scratch);
  auto mrg_acc = reinterpret_cast<float (*)[RW][D]>(scratch);

  const int tid = threadIdx.x;
  // The wave index is uniform across the wave; saying so keeps the key loop's
  // control flow scalar (a per-lane loop exit would copy the accumulators out
  // of the matrix-core registers on every block).
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;
  // Workgroup = (sequence, group of up to RW of its query rows, key split).
  const int64_t seq = blockIdx.x / p.rgroups;
  const int r0 = RW * (int)(blockIdx.x % p.rgroups);
  const int split = blockIdx.y;
  const int64_t b_ = seq / p.Hkv;
  const int hkv = (int)(seq % p.Hkv);
  const int G = p.Hq / p.Hkv;
  const int rows = min(RW, G * p.Tq - r0);  // query rows of this workgroup
  auto qrow_of = [&](int r) -> int64_t {
    const int rr = r0 + r;  // row within the KV head's G * Tq rows
    return (b_ * p.Hq + (int64_t)hkv * G + rr / p.Tq) * p.Tq + rr % p.Tq;
  };

  SeqBuffers sb;
  sb.kidx = make_rsrc(p.kidx + seq * p.cap * S::KROW, p.cap * S::KROW);
  sb.ksign = make_rsrc(QJL ? p.ksign + seq * p.cap * (D / 8) : p.kidx, p.cap * (D / 8));
  sb.knorm = make_rsrc(p.knorm + seq * p.cap, p.N * 4);
  sb.krnorm = make_rsrc(QJL ? p.krnorm + seq * p.cap : p.knorm, p.N * 4);
  sb.vidx = make_rsrc(p.vidx + seq * (p.cap / 8) * S::VTILE, (p.cap / 8) * S::VTILE);
  sb.vnorm = make_rsrc(p.vnorm + seq * p.cap, p.N * 4);

  // The split's key blocks [blk0, blk1): wave w takes blocks blk0 + w + W j.
  // The first ones start loading before the set-up below (two at d = 128, one
  // at d = 256, whose loop keeps two register sets).
  int blk0, blk1;
  split_blocks(p, split, blk0, blk1);
  Block<D, KB, QJL, VB> b0, b1, b2;
  int blk = blk0 + wave;
  load_block(b0, sb, blk * 32, l16, g4);
  if constexpr (D == 128) load_block(b1, sb, (blk + W) * 32, l16, g4);

  WaveState<D, KB, QJL, VB, NR> ws;
  const float scale_k = p.scales[0], scale_v = KB == VB ? scale_k : p.scales[1];
  if constexpr (TB::kColK)
    fill_lut_cols4<T>(lut, p.cb, scale_k, tid);
  else
    fill_lut<KB, T>(lut, p.cb, scale_k, tid);
  if constexpr (KB != VB) {
    if constexpr (TB::kColV)
      fill_lut_cols4<T>(lut + TB::kK, p.cb + 2 * kMaxLevels, scale_v, tid);
    else
      fill_lut<VB, T>(lut + TB::kK, p.cb + 2 * kMaxLevels, scale_v, tid);
  }
  ws.ktab = lut;
  ws.vtab = KB == VB ? lut : lut + TB::kK;
  ws.kcol = ws.ktab + lane % 32;
  ws.vcol = ws.vtab + lane % 32;

  // Rotate the query rows once (R q, S q) and normalise them for the fp16
  // operand split: qa = (R q) / (s_k c1), qb = 2 (S q) / c2 with c1, c2 powers of
  // two that bring the largest entry into [1, 2).
  for (int i = tid; i < RW * D; i += T) {
    const int r = i / D, k = i % D;
    float v = 0.f;
    if (r < rows) {
      const int64_t o = qrow_of(r) * D + k;
      v = p.qdt == TQ_F16 ? __half2float(static_cast<const __half*>(p.q)[o]) : static_cast<const float*>(p.q)[o];
    }
    qsh[r][k] = v;
  }
  __syncthreads();  // also publishes the code tables
  {
    const int k0 = (int)((blockIdx.x * 5 + blockIdx.y * 3) * 16) & (D - 1);
#pragma unroll
    for (int rb = 0; rb < RW; rb += 4) {
      if (rb > 0) __syncthreads();  // rpart is reused
      rotate_rows<D, QJL, RW, T>(p.Rt, p.St, scale_k, qsh, qrs, rpart, tid, k0, rb);
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = wave; r < RW; r += W) {  // wave w normalises rows w, w + W, ...
    float ma = 0.f, mb = 0.f, sbv = 0.f, sav = 0.f;
#pragma unroll
    for (int j = lane; j < D; j += 64) {
      ma = fmaxf(ma, fabsf(qrs[0][r][j]));
      if constexpr (DITHER) sav += qrs[0][r][j];
      if constexpr (QJL) {
        mb = fmaxf(mb, fabsf(qrs[1][r][j]));
        sbv += qrs[1][r][j];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      ma = fmaxf(ma, __shfl_xor(ma, o));
      mb = fmaxf(mb, __shfl_xor(mb, o));
      sbv += __shfl_xor(sbv, o);
      if constexpr (DITHER) sav += __shfl_xor(sav, o);
    }
    if (lane == 0) {
      int e1 = 0, e2 = 0;
      frexpf(ma, &e1);
      frexpf(mb, &e2);
      qcon[r][0] = ma > 0.f ? ldexpf(1.f, e1 - 1) : 1.f;
      qcon[r][1] = mb > 0.f ? ldexpf(1.f, e2) : 2.f;
      qcon[r][2] = QJL ? -sbv : 0.f;
      qcon[r][3] = sav * scale_k;  // qrs[0] holds R q / s_k
    }
  }
  __syncthreads();

  // Query operands: lane (row rho = l16, k-group g4).  NR = 1: rho = 4 qr + part,
  // parts {R q hi, R q lo} in Ak and {S q hi, S q lo} in As; NR = 2: rho = 2 qr +
  // part, parts {hi, lo} in both.  Every lane reads and scales its values (qr <
  // RW keeps the reads inside qrs, whose rows are finite), the factor being 0
  // for lanes outside the rows and parts: a read used only under that condition
  // compiles into one branch and one full LDS wait per element.
  {
    const int qr = NR == 1 ? l16 / 4 : l16 / 2, part = NR == 1 ? l16 % 4 : l16 % 2;
    const bool ok = qr < rows;
    const float fa = 1.0f / qcon[qr][0], fb = 2.0f / qcon[qr][1];  // powers of two: exact
    const float* qa = &qrs[0][qr][(D / 4) * g4];
    const float* qb = &qrs[1][qr][(D / 4) * g4];
    sfor<0, S::KBLK>([&](auto kb) {
      h8 a;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qa[8 * kb + e] * ((ok && part < 2) ? fa : 0.f);  // NR = 2: part < 2 always
        const _Float16 hi = (_Float16)x;
        const _Float16 lo = (_Float16)(x - (float)hi);
        a[e] = part == 0 ? hi : (part == 1 ? lo : (_Float16)0.f);
      }
      ws.Ak[kb] = a;
      if constexpr (QJL) {
        h8 s;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e / 2, h = e % 2;
          const bool sp = NR == 1 ? part >= 2 : true;  // rows of the sign term
          const float x = qb[32 * (kb / 4) + sign_coord(kb % 4, w, h)] * ((ok && sp) ? fb * sign_comp(w) : 0.f);
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)(x - (float)hi);
          const int sp_part = NR == 1 ? part - 2 : part;
          s[e] = sp_part == 0 ? hi : (sp_part == 1 ? lo : (_Float16)0.f);
        }
        ws.As[kb] = s;
      }
    });
  }
  // Score-side constants of this lane's query rows NR g4 + j (log2 domain).
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int q = NR * g4 + j;
    ws.ca[j] = ws.c2[j] = ws.c0[j] = ws.cd[j] = ws.dacc[j] = 0.f;
    ws.limit[j] = -1;
    ws.srow[j] = 0;
    if (q < rows) {
      ws.srow[j] = qrow_of(q);
      const float* rc = qcon[q];
      const float inv_sqrt_d = 1.0f / sqrtf((float)D);
      const float cq = sqrtf(0.5f * (float)M_PI) / (float)D * inv_sqrt_d * kLog2e;
      ws.ca[j] = rc[0] * inv_sqrt_d * kLog2e;
      ws.c2[j] = rc[1] * cq;
      ws.c0[j] = rc[2] * cq;
      ws.cd[j] = rc[3] * inv_sqrt_d * kLog2e;
      ws.limit[j] = (int)(p.causal ? p.N - p.Tq + ((r0 + q) % p.Tq) + 1 : p.N);
    }
    ws.m[j] = -INFINITY;
    ws.msafe[j] = 0.f;
    ws.lsum[j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < S::CB; ++i) ws.acc[i] = f4{0.f, 0.f, 0.f, 0.f};
  ws.vsc = kInvSlack;
  ws.vlim = ldexpf(1.f, kVExp) / kInvSlack;
  ws.seq = seq;
  ws.dkw = DITHER ? p.scales[4] : 0.f;
  ws.dvw = DITHER ? p.scales[5] : 0.f;

  // Three register sets rotate so two blocks are in flight while one is used
  // (d = 256: two sets, one block in flight).  The prefetches are
  // unconditional (reads past the split land in the same sequence, reads past
  // its capacity return 0), which keeps the loop body straight-line and lets
  // the compiler count outstanding loads exactly.
  if constexpr (D == 128) {
    for (; blk < blk1; blk += 3 * W) {
      load_block(b2, sb, (blk + 2 * W) * 32, l16, g4);
      process_block<D, KB, QJL, VB, SCORES, NR, DITHER>(ws, b0, blk * 32, p, pbuf[wave], l16, g4, rows);
      if (blk + W >= blk1) break;
      load_block(b0, sb, (blk + 3 * W) * 32, l16, g4);
      process_block<D, KB, QJL, VB, SCORES, NR, DITHER>(ws, b1, (blk + W) * 32, p, pbuf[wave], l16, g4, rows);
      if (blk + 2 * W >= blk1) break;
      load_block(b1, sb, (blk + 4 * W) * 32, l16, g4);
      process_block<D, KB, QJL, VB, SCORES, NR, DITHER>(ws, b2, (blk + 2 * W) * 32, p, pbuf[wave], l16, g4, rows);
    }
  } else {
    for (; blk < blk1; blk += 2 * W) {
      load_block(b1, sb, (blk + W) * 32, l16, g4);
      process_block<D, KB, QJL, VB, SCORES, NR, DITHER>(ws, b0, blk * 32, p, pbuf[wave], l16, g4, rows);
      if (blk + W >= blk1) break;
      load_block(b0, sb, (blk + 2 * W) * 32, l16, g4);
      process_block<D, KB, QJL, VB, SCORES, NR, DITHER>(ws, b1, (blk + W) * 32, p, pbuf[wave], l16, g4, rows);
    }
  }

  // Merge the waves of this workgroup.
  __syncthreads();  // mrg_acc shares its memory with the set-up's rotation buffer
  const float inv_sv = 1.f / (ws.vsc * scale_v);  // undoes the value-norm and fp16 table factors
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float lsum = ws.lsum[j];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) lsum += __shfl_xor(lsum, o);
    if (l16 == 0) {
      mrg_m[wave][NR * g4 + j] = ws.m[j];
      mrg_l[wave][NR * g4 + j] = lsum;
    }
    float dsum = 0.f;  // the value offsets' share of every coordinate
    if constexpr (DITHER) {
      dsum = ws.dacc[j];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) dsum += __shfl_xor(dsum, o);
    }
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
      mrg_acc[wave][NR * g4 + j][l16 * S::CB + cb] = fmaf(ws.acc[cb][2 * j] + ws.acc[cb][2 * j + 1], inv_sv, dsum);
  }
  __syncthreads();
  const int64_t rows_total = (int64_t)(gridDim.x / p.rgroups) / p.Hkv * p.Hq * p.Tq;
  for (int idx = tid; idx < rows * D; idx += T) {
    const int r = idx / D, j = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, mrg_m[w][r]);
    float a = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = exp2f(mrg_m[w][r] - M);
        a = fmaf(f, mrg_acc[w][r][j], a);
        L = fmaf(f, mrg_l[w][r], L);
      }
    }
    float* dst = p.part + ((int64_t)split * rows_total + qrow_of(r)) * (D + kPartPad);
    dst[j] = a;
    if (j == 0) {
      dst[D] = M * kLn2;  // natural-log units, as the combine kernel expects
      dst[D + 1] = L;
    }
  }
}

}  // namespace
}  // namespace tq
