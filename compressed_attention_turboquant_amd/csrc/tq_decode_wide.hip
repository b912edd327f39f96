// Decode on the matrix cores for KV heads with many query rows (d = 128):
// grouped-query heads times chunked query tokens, e.g. 8 query heads x 16
// tokens = 128 rows sharing every key of a KV head.
//
// Same computation as the split kernel of tq_decode_mfma_impl.h ([cuTile]
// listing: asymmetric score estimator, fused attention with online softmax and
// values decoded on chip; [Mobilint] "Two-Stage Approach": <q, x~> = <Pi q, y~>),
// organised so that each decoded code serves 32 query rows:
//  * A workgroup of 4 waves serves up to 64 query rows of one KV head and one
//    key split; each wave owns 16 rows (one column tile; two with
//    TQ_WIDE_CT=2) and walks all of the split's 32-key blocks.  A block's
//    codes are decoded (LDS table lookups) once per wave, i.e. once per 16 rows
//    instead of once per 4 or 8.
//  * Scores are computed transposed, S^T = K Q^T: the decoded keys are the A
//    operand (16 keys x 32 coordinates) and the query rows the B operand, so a
//    lane ends with 8 keys of one query row -- exactly the A operand layout of
//    the P.V product.  With lane l16 of tile t holding key
//    8 (l16 / 4) + 4 t + l16 % 4, lane group g4 gets keys 8 g4 .. 8 g4 + 7,
//    the 8 tokens of value tile g4: P never leaves the registers.
//  * The query rows are rotated on the matrix cores in the prologue (R q from
//    sqrt(d) R and S q from S, both split fp16 hi + lo; q fp16 is exact, fp32 q
//    is split too).  The rows of R and S are taken in the order that makes the
//    product land directly in the B operand layout of the score products (lane
//    group g4 holds the quarter 32 g4 .. 32 g4 + 31 of the coordinates, which
//    is the quarter of a key's code stream it decodes: 32 g4 + 8 kb + e for the
//    centroid term, the masked-exponent order for the sign term).
//  * hi and lo parts of the query (and of p) are separate products into one
//    accumulator; the softmax runs per query row with the lazily updated
//    maximum and value-norm scale of the split kernel.
// Each wave writes its rows' split partials; the combine kernel merges splits.
#include "tq_decode_mfma_impl.h"

#if !defined(TQ_INST_QJL)
#error "compile with -DTQ_INST_QJL=<0|1>"
#endif

namespace tq {
namespace {

constexpr int kWD = 128;      // head dimension
constexpr int kWW = 4;        // waves per workgroup

template <int KB, int QJL, int VB>
struct WideBlock {
  using S = Shape<kWD, KB, QJL, VB>;
  uint32_t kw[2][S::NWK];  // codes of key(t, l16), this lane's quarter of the coordinates
  uint32_t sw[2][1];       // sign dword g4 of key(t, l16)
  f4 kn[2], kg[2], vn[2];  // norms of keys 8 g4 + 4 t + i
  uint32_t vw[S::NWV];     // value tile g4: coordinates 8 l16 .. 8 l16 + 7
};

template <int KB, int QJL, int VB>
__device__ __forceinline__ void load_wide(WideBlock<KB, QJL, VB>& b, const SeqBuffers& sb, int k0, int l16,
                                          int g4) {
  using S = Shape<kWD, KB, QJL, VB>;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = k0 + 8 * (l16 >> 2) + 4 * t + (l16 & 3);
    buf_load(b.kw[t], sb.kidx, key * S::KROW + g4 * (S::KROW / 4));
    if constexpr (QJL) buf_load(b.sw[t], sb.ksign, key * (kWD / 8) + g4 * 4);
  }
  const int nb = (k0 + 8 * g4) * 4;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    b.kn[t] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(sb.knorm, nb + 16 * t, 0, 0));
    if constexpr (QJL)
      b.kg[t] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(sb.krnorm, nb + 16 * t, 0, 0));
    b.vn[t] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(sb.vnorm, nb + 16 * t, 0, 0));
  }
  buf_load(b.vw, sb.vidx, (int)__umul24((unsigned)(k0 / 8 + g4), (unsigned)S::VTILE) + l16 * (S::VTILE / 16));
}

// Per-wave state: query operands, softmax state and accumulators of the
// wave's two 16-row column tiles (lane l16 of tile ct is query row 16 ct + l16
// of the wave's rows; accumulator rows 4 g4 + r are rows 16 ct + 4 g4 + r).
template <int QJL, int CT>
struct WideState {
  h8 bqh[CT][4], bql[CT][4];                         // centroid term, hi and lo
  h8 bsh[QJL ? CT : 1][4], bsl[QJL ? CT : 1][4];     // sign term, hi and lo
  f4 acc[CT][8];                                     // P.V, rotated domain
  // Scores are kept in units of 1/ca (ca: the row's factor to log2 units), the
  // factor applied in the exponent's FMA: s = kn (sc + kg r2 ss), with the
  // sign product ss started at r0 (the offset of the masked-exponent operand).
  // The value-norm factor vsc (a power of two) rides in the exponent: cm =
  // log2(vsc) - ca * max, so the weights and lsum carry it too.
  float m[CT], cm[CT], sl[CT], lsum[CT], ca[CT], r2[CT], r0[CT];  // sl = kSlack / ca
  int limit[CT];
  float vsc, vlim, lv;  // lv = log2(vsc)
  const uint32_t *ktab, *vtab;
};

// MASK: the block may hold keys at or past N or past a row's causal limit
// (the tail of a split); other blocks skip those selects.
template <int KB, int QJL, int VB, int SCORES, int CT, bool MASK>
__device__ __forceinline__ void process_wide(WideState<QJL, CT>& ws, const WideBlock<KB, QJL, VB>& cur, int k0,
                                             const DecodeMfmaParams& p, const int64_t (&srow)[CT], int l16,
                                             int g4) {
  const int N = (int)p.N;  // below 2^31: caches hold less than 2^31 bytes per sequence
  f4 sc[2][CT], ss[2][CT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      sc[t][ct] = f4{0.f, 0.f, 0.f, 0.f};
      ss[t][ct] = f4{ws.r0[ct], ws.r0[ct], ws.r0[ct], ws.r0[ct]};
    }
  // Scores: decoded keys (A) times the query rows' hi and lo parts (B).
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u4 ak[4];
    sfor<0, 4>([&](auto kb) { ak[kb] = decode8<KB, 8 * KB * kb>(cur.kw[t], ws.ktab); });
    __builtin_amdgcn_sched_barrier(0);
    sfor<0, 4>([&](auto kb) {
      const h8 a = __builtin_bit_cast(h8, ak[kb]);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        sc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ws.bqh[ct][kb], sc[t][ct], 0, 0, 0);
        sc[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ws.bql[ct][kb], sc[t][ct], 0, 0, 0);
      }
      if constexpr (QJL) {
        constexpr int r = decltype(kb)::value % 4;
        const uint32_t word = cur.sw[t][0];
        const uint32_t rot = r == 0 ? word : __builtin_amdgcn_alignbit(word, word, 32 - 4 * r);
        u4 bw;
        sfor<0, 4>([&](auto w) { bw[decltype(w)::value] = sign_dword<decltype(w)::value>(rot); });
        const h8 as = __builtin_bit_cast(h8, bw);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          ss[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as, ws.bsh[ct][kb], ss[t][ct], 0, 0, 0);
          ss[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as, ws.bsl[ct][kb], ss[t][ct], 0, 0, 0);
        }
      }
    });
  }
  // First half of the value operands: their table lookups are in flight
  // during the softmax.
  u4 bv[4];
  sfor<0, 4>([&](auto cb) { bv[cb] = decode8<VB, 8 * VB * cb>(cur.vw, ws.vtab); });
  __builtin_amdgcn_sched_barrier(0);

  // Value norms of the lane's keys; keys at or past N carry weight 0 and their
  // norm words may hold anything, so they count as 0.  Key indices are taken
  // relative to the lane's first key: keys below nrel exist, keys below lrel
  // are visible to the row (one subtraction per block, not an addition per key).
  const int kbase = k0 + 8 * g4;
  const int nrel = N - kbase;
  float vnv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) vnv[e] = !MASK || e < nrel ? cur.vn[e / 4][e % 4] : 0.f;
  // Value-norm scale (as in the split kernel): the block's largest norm over
  // the lane's 8 keys and the four lane groups.  The norms are >= 0, so their
  // bit patterns order like the values (integer maxima, no NaN handling).
  {
    uint32_t vb = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) vb = max(vb, __float_as_uint(vnv[e]));
    float vl = __uint_as_float(vb);
    if (__any(vl > ws.vlim)) {
      vl = max_over_row_groups(vl);
      int e = 0;
      frexpf(vl, &e);
      const float nlv = fminf(ws.lv, (float)(kVExp - e));
      const float nsc = ldexpf(1.f, (int)nlv);
      const float ratio = nsc / ws.vsc;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) ws.acc[ct][cb] *= ratio;
        ws.lsum[ct] *= ratio;
        ws.cm[ct] += nlv - ws.lv;
      }
      ws.vsc = nsc;
      ws.lv = nlv;
      ws.vlim = ldexpf(1.f, kVExp) / nsc;
    }
  }

  h8 ph[CT], pl[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int lrel = ws.limit[ct] - kbase;
    float s[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v;
        if constexpr (QJL) v = cur.kn[t][i] * fmaf(cur.kg[t][i] * ws.r2[ct], ss[t][ct][i], sc[t][ct][i]);
        else v = cur.kn[t][i] * sc[t][ct][i];
        if constexpr (MASK) v = 4 * t + i < lrel ? v : -INFINITY;
        if constexpr (SCORES) {
          if (ws.limit[ct] >= 0 && 4 * t + i < nrel)
            p.scores[srow[ct] * p.N + kbase + 4 * t + i] = v * (ws.ca[ct] * kLn2);
        }
        s[4 * t + i] = v;
      }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = max_over_row_groups(mx);
    if (__any(mx > ws.m[ct] + ws.sl[ct])) {
      const float mnew = fmaxf(ws.m[ct], mx);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(ws.ca[ct] * (ws.m[ct] - mnew));
      ws.lsum[ct] *= alpha;
      float ar[4];  // factors of the accumulator rows 4 g4 + r (held by lanes l16 = 4 g4 + r)
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g4 + r);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) ws.acc[ct][cb][r] *= ar[r];
      ws.m[ct] = mnew;
      ws.cm[ct] = mnew == -INFINITY ? ws.lv : fmaf(-ws.ca[ct], mnew, ws.lv);
    }
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * t + i;
        const float pr = __builtin_amdgcn_exp2f(fmaf(ws.ca[ct], s[e], ws.cm[ct]));
        ls += pr;
        const float q = pr * vnv[e];
        const _Float16 h = (_Float16)q;
        ph[ct][e] = h;
        pl[ct][e] = (_Float16)(q - (float)h);
      }
    ws.lsum[ct] += ls;
  }
  // P.V: A = p (hi, lo) of the lane's query row, B = decoded values; the
  // second half of the values is decoded while the first half's products run.
  sfor<0, 4>([&](auto cb) {
    const h8 b = __builtin_bit_cast(h8, bv[cb]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      ws.acc[ct][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[ct], b, ws.acc[ct][cb], 0, 0, 0);
      ws.acc[ct][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[ct], b, ws.acc[ct][cb], 0, 0, 0);
    }
  });
  sfor<0, 4>([&](auto cb) { bv[cb] = decode8<VB, 8 * VB * (cb + 4)>(cur.vw, ws.vtab); });
  sfor<0, 4>([&](auto cb) {
    const h8 b = __builtin_bit_cast(h8, bv[cb]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      ws.acc[ct][cb + 4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[ct], b, ws.acc[ct][cb + 4], 0, 0, 0);
      ws.acc[ct][cb + 4] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[ct], b, ws.acc[ct][cb + 4], 0, 0, 0);
    }
  });
}

// CT: 16-row column tiles per wave (2: one wave per SIMD; 1: two).
template <int KB, int QJL, int VB, int SCORES, int CT>
__global__ void __launch_bounds__(64 * kWW) __attribute__((amdgpu_waves_per_eu(3 - CT, 3 - CT)))
decode_wide_kernel(DecodeMfmaParams p) {
  constexpr int kRowsWave = 16 * CT;
  using S = Shape<kWD, KB, QJL, VB>;
  constexpr int T = 64 * kWW;
  constexpr int kKtab = Lut<KB>::kDwords, kVtab = KB == VB ? 0 : Lut<VB>::kDwords;
  __shared__ __align__(16) uint32_t lut[kKtab + kVtab];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int l16 = lane % 16, g4 = lane / 16;
  // Workgroup -> (sequence, row group).  Workgroups are dealt to the eight
  // XCDs in turn by their linear index, and each XCD has its own L2: the row
  // groups of one sequence read the same keys, so they are given indices eight
  // apart (same XCD, running at about the same time), and the second finds
  // the keys in L2.  This needs the sequence count to be a multiple of 8 (the
  // row of workgroups of one split then starts on XCD 0); else the plain order.
  const int nseq = (int)gridDim.x / p.rgroups;
  int64_t seq;
  int rg;
  if (p.rgroups > 1 && nseq % 8 == 0) {
    const int x = (int)blockIdx.x, slot = x / 8;
    rg = slot % p.rgroups;
    seq = (int64_t)(slot / p.rgroups) * 8 + x % 8;
  } else {
    seq = blockIdx.x / p.rgroups;
    rg = (int)(blockIdx.x % p.rgroups);
  }
  const int split = blockIdx.y;
  const int64_t b_ = seq / p.Hkv;
  const int hkv = (int)(seq % p.Hkv);
  const int G = p.Hq / p.Hkv;
  const int RH = G * p.Tq;  // query rows of the KV head
  const int row0 = rg * (kWW * kRowsWave) + kRowsWave * wave;
  static_assert(kWW * kRowsWave == kWideRowsPerGroup, "row group size");
  auto qrow_of = [&](int c) -> int64_t { return (b_ * p.Hq + (int64_t)hkv * G + c / p.Tq) * p.Tq + c % p.Tq; };

  SeqBuffers sb;
  sb.kidx = make_rsrc(p.kidx + seq * p.cap * S::KROW, p.cap * S::KROW);
  sb.ksign = make_rsrc(QJL ? p.ksign + seq * p.cap * (kWD / 8) : p.kidx, p.cap * (kWD / 8));
  sb.knorm = make_rsrc(p.knorm + seq * p.cap, p.N * 4);
  sb.krnorm = make_rsrc(QJL ? p.krnorm + seq * p.cap : p.knorm, p.N * 4);
  sb.vidx = make_rsrc(p.vidx + seq * (p.cap / 8) * S::VTILE, (p.cap / 8) * S::VTILE);
  sb.vnorm = make_rsrc(p.vnorm + seq * p.cap, p.N * 4);

  int blk0, blk1;
  split_blocks(p, split, blk0, blk1);
  WideBlock<KB, QJL, VB> b0, b1;
  int blk = blk0;
  load_wide(b0, sb, blk * 32, l16, g4);

  WideState<QJL, CT> ws;
  const float scale_k = p.scales[0], scale_v = KB == VB ? scale_k : p.scales[1];
  fill_lut<KB, T>(lut, p.cb, scale_k, tid);
  if constexpr (KB != VB) fill_lut<VB, T>(lut + kKtab, p.cb + 2 * kMaxLevels, scale_v, tid);
  ws.ktab = lut;
  ws.vtab = KB == VB ? lut : lut + kKtab;

  // ---- Query rows on the matrix cores: v = sqrt(d) R q and S q. ----
  // B operand: query row 16 ct + l16 of the wave, input coordinates 32 kk + 8 g4 + e.
  int64_t srow[CT];
  {
    h8 qh[CT][4], ql[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c = row0 + 16 * ct + l16;
      const bool ok = c < RH;
      srow[ct] = ok ? qrow_of(c) : 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        h8 h = h8{0, 0, 0, 0, 0, 0, 0, 0}, l = h;
        if (ok) {
          const int64_t o = srow[ct] * kWD + 32 * kk + 8 * g4;
          if (p.qdt == TQ_F16) {
            h = *reinterpret_cast<const h8*>(static_cast<const _Float16*>(p.q) + o);
          } else {
            const f4* src = reinterpret_cast<const f4*>(static_cast<const float*>(p.q) + o);
            const f4 x0 = src[0], x1 = src[1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = e < 4 ? x0[e] : x1[e - 4];
              h[e] = (_Float16)x;
              l[e] = (_Float16)(x - (float)h[e]);
            }
          }
        }
        qh[ct][kk] = h;
        ql[ct][kk] = l;
      }
    }
    const bool q32 = p.qdt != TQ_F16;
    const _Float16* Rh = static_cast<const _Float16*>(p.rot_hi);
    const _Float16* Rl = static_cast<const _Float16*>(p.rot_lo);
    const _Float16* Sh = static_cast<const _Float16*>(p.proj_hi);
    const _Float16* Sl = static_cast<const _Float16*>(p.proj_lo);
    f4 rq[CT][4][2], sq[CT][4][2];  // [ct][kb][hf]: coordinates 32 g4 + 8 kb + 4 hf + r (sign order for sq)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int rowR = 32 * (l16 >> 2) + 8 * kb + 4 * hf + (l16 & 3);
        const int e = 4 * hf + (l16 & 3), w = e >> 1, h = e & 1;
        const int rowS = 32 * (l16 >> 2) + ((10 + w + 16 * h - 4 * kb) & 31);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) rq[ct][kb][hf] = sq[ct][kb][hf] = f4{0.f, 0.f, 0.f, 0.f};
        // hi x hi and lo x hi products, plus hi x lo for fp32 queries (the
        // branch is uniform and taken once, outside the products).
        auto products = [&](auto with_lo) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int col = 32 * kk + 8 * g4;
            const h8 ah = *reinterpret_cast<const h8*>(Rh + rowR * kWD + col);
            const h8 al = *reinterpret_cast<const h8*>(Rl + rowR * kWD + col);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              rq[ct][kb][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qh[ct][kk], rq[ct][kb][hf], 0, 0, 0);
              rq[ct][kb][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qh[ct][kk], rq[ct][kb][hf], 0, 0, 0);
              if constexpr (decltype(with_lo)::value)
                rq[ct][kb][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ql[ct][kk], rq[ct][kb][hf], 0, 0, 0);
            }
            if constexpr (QJL) {
              const h8 sh = *reinterpret_cast<const h8*>(Sh + rowS * kWD + col);
              const h8 sl = *reinterpret_cast<const h8*>(Sl + rowS * kWD + col);
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) {
                sq[ct][kb][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sh, qh[ct][kk], sq[ct][kb][hf], 0, 0, 0);
                sq[ct][kb][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sl, qh[ct][kk], sq[ct][kb][hf], 0, 0, 0);
                if constexpr (decltype(with_lo)::value)
                  sq[ct][kb][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sh, ql[ct][kk], sq[ct][kb][hf], 0, 0, 0);
              }
            }
          }
        };
        if (q32)
          products(std::integral_constant<bool, true>{});
        else
          products(std::integral_constant<bool, false>{});
      }
    // Normalise each row for the fp16 split: the centroid part by a power of
    // two c1 (and the table factor), the sign part by 2 / c2 and the masked-
    // exponent factors.  The four lane groups of a row combine their maxima.
    const float inv_sqrt_d = 1.0f / sqrtf((float)kWD);
    const float cq = sqrtf(0.5f * (float)M_PI) / (float)kWD * inv_sqrt_d * kLog2e;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float ma = 0.f, mb = 0.f, sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ma = fmaxf(ma, fabsf(rq[ct][kb][hf][r]));
            if constexpr (QJL) {
              mb = fmaxf(mb, fabsf(sq[ct][kb][hf][r]));
              sum += sq[ct][kb][hf][r];
            }
          }
      ma = fmaxf(ma, __shfl_xor(ma, 16));
      ma = fmaxf(ma, __shfl_xor(ma, 32));
      mb = fmaxf(mb, __shfl_xor(mb, 16));
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      int e1 = 0, e2 = 0;
      frexpf(ma, &e1);
      frexpf(mb, &e2);
      const float c1 = ma > 0.f ? ldexpf(1.f, e1 - 1) : 1.f;
      const float c2v = mb > 0.f ? ldexpf(1.f, e2) : 2.f;
      const float fa = 1.f / c1, fb = 2.f / c2v;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        h8 hi, lo, shi, slo;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * hf + r;
            const float x = (rq[ct][kb][hf][r] / scale_k) * fa;
            hi[e] = (_Float16)x;
            lo[e] = (_Float16)(x - (float)hi[e]);
            if constexpr (QJL) {
              const float y = sq[ct][kb][hf][r] * (fb * sign_comp(e >> 1));
              shi[e] = (_Float16)y;
              slo[e] = (_Float16)(y - (float)shi[e]);
            }
          }
        ws.bqh[ct][kb] = hi;
        ws.bql[ct][kb] = lo;
        if constexpr (QJL) {
          ws.bsh[ct][kb] = shi;
          ws.bsl[ct][kb] = slo;
        }
      }
      // v = sqrt(d) R q, so the centroid product carries sqrt(d) / c1 on top
      // of R q: c1 / sqrt(d) undoes it, and 1 / sqrt(d) is the score's factor.
      ws.ca[ct] = c1 * inv_sqrt_d * inv_sqrt_d * kLog2e;
      // sign term c2v cq (ss + r0) with ss the product of the normalised
      // operand; offset r0 = -sum / c2v; in units of 1/ca
      ws.r2[ct] = c2v * cq / ws.ca[ct];
      ws.r0[ct] = -sum / c2v;
      ws.sl[ct] = kSlack / ws.ca[ct];
      const int c = row0 + 16 * ct + l16;
      ws.limit[ct] = c < RH ? (int)(p.causal ? p.N - p.Tq + (c % p.Tq) + 1 : p.N) : -1;
      ws.m[ct] = -INFINITY;
      ws.cm[ct] = -kSlack;  // log2(kInvSlack), the initial vsc
      ws.lsum[ct] = 0.f;
    }
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) ws.acc[ct][cb] = f4{0.f, 0.f, 0.f, 0.f};
  ws.vsc = kInvSlack;
  ws.lv = -kSlack;
  ws.vlim = ldexpf(1.f, kVExp) / kInvSlack;
  __syncthreads();  // the code tables are filled

  // Two rotating register sets, one block in flight while the other is used
  // (a block's matrix-core work covers the load latency).  Prefetches past the
  // split stay inside the sequence (or return 0 past its capacity).
  // Blocks wholly below N and below every row's causal limit (at least
  // N - Tq + 1) need no masks: pairs of them first, then the rest masked.
  const int64_t unmasked_end = p.causal ? p.N - p.Tq + 1 : p.N;  // keys [0, unmasked_end) are visible to every row
  int mid = (int)min((int64_t)blk1, unmasked_end / 32);
  mid = mid <= blk ? blk : blk + ((mid - blk) & ~1);
  for (; blk < mid; blk += 2) {
    load_wide(b1, sb, (blk + 1) * 32, l16, g4);
    process_wide<KB, QJL, VB, SCORES, CT, false>(ws, b0, blk * 32, p, srow, l16, g4);
    load_wide(b0, sb, (blk + 2) * 32, l16, g4);
    process_wide<KB, QJL, VB, SCORES, CT, false>(ws, b1, (blk + 1) * 32, p, srow, l16, g4);
  }
  for (; blk < blk1; blk += 2) {
    load_wide(b1, sb, (blk + 1) * 32, l16, g4);
    process_wide<KB, QJL, VB, SCORES, CT, true>(ws, b0, blk * 32, p, srow, l16, g4);
    if (blk + 1 >= blk1) break;
    load_wide(b0, sb, (blk + 2) * 32, l16, g4);
    process_wide<KB, QJL, VB, SCORES, CT, true>(ws, b1, (blk + 1) * 32, p, srow, l16, g4);
  }

  // Partials of the wave's rows: accumulator rows 4 g4 + r of each tile hold
  // coordinates 8 l16 + cb; (max, sum) of row l16 come from the lanes with g4 = 0.
  const int64_t rows_total = (int64_t)(gridDim.x / p.rgroups) / p.Hkv * p.Hq * p.Tq;
  const float inv_sv = 1.f / (ws.vsc * scale_v);
  const float inv_vsc = 1.f / ws.vsc;  // exact: a power of two
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float L = sum_over_row_groups(ws.lsum[ct]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = row0 + 16 * ct + 4 * g4 + r;
      if (c < RH) {
        float* dst = p.part + ((int64_t)split * rows_total + qrow_of(c)) * (kWD + kPartPad) + 8 * l16;
        const f4 a0 = {ws.acc[ct][0][r], ws.acc[ct][1][r], ws.acc[ct][2][r], ws.acc[ct][3][r]};
        const f4 a1 = {ws.acc[ct][4][r], ws.acc[ct][5][r], ws.acc[ct][6][r], ws.acc[ct][7][r]};
        reinterpret_cast<f4*>(dst)[0] = a0 * inv_sv;
        reinterpret_cast<f4*>(dst)[1] = a1 * inv_sv;
      }
    }
    const int c = row0 + 16 * ct + l16;
    if (g4 == 0 && c < RH) {
      float* dst = p.part + ((int64_t)split * rows_total + qrow_of(c)) * (kWD + kPartPad);
      dst[kWD] = ws.m[ct] * (ws.ca[ct] * kLn2);  // natural-log units, as the combine kernel expects
      dst[kWD + 1] = L * inv_vsc;
    }
  }
}

template <int KB, int QJL, int VB>
hipError_t launch_wide(const DecodeMfmaParams& p, dim3 grid, hipStream_t st) {
  if (p.scores)
    hipLaunchKernelGGL((decode_wide_kernel<KB, QJL, VB, 1, kWideCT>), grid, dim3(64 * kWW), 0, st, p);
  else
    hipLaunchKernelGGL((decode_wide_kernel<KB, QJL, VB, 0, kWideCT>), grid, dim3(64 * kWW), 0, st, p);
  return hipGetLastError();
}

template <int KB, int QJL>
hipError_t wide_vb(const DecodeMfmaParams& p, int vb, dim3 grid, hipStream_t st) {
  switch (vb) {
    case 1: return launch_wide<KB, QJL, 1>(p, grid, st);
    case 2: return launch_wide<KB, QJL, 2>(p, grid, st);
    case 3: return launch_wide<KB, QJL, 3>(p, grid, st);
    default: return launch_wide<KB, QJL, 4>(p, grid, st);
  }
}

}  // namespace

template <>
hipError_t launch_decode_wide<TQ_INST_QJL>(const DecodeMfmaParams& p, int kb, int vb, dim3 grid, hipStream_t st) {
  switch (kb) {
    case 1: return wide_vb<1, TQ_INST_QJL>(p, vb, grid, st);
    case 2: return wide_vb<2, TQ_INST_QJL>(p, vb, grid, st);
    case 3: return wide_vb<3, TQ_INST_QJL>(p, vb, grid, st);
    default: return wide_vb<4, TQ_INST_QJL>(p, vb, grid, st);
  }
}

}  // namespace tq
