// Fused decode attention over the quantized page records (gfx950).
//
// "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with Dynamic
// Channel-wise Precision Boost", Abstract: the page dequantization is uniform
// across lanes because each mixed-precision Key page is two uniform 2-bit
// tensors.  Here the dequantization is folded into the two contractions:
//
//   q . k^_t = sum_c (q_c kscale_c) base_tc + sum_j (q_idx_j kscale_idx_j / 4)
//              boost_tj + sum_c q_c kmin_c
//   sum_t p_t v^_tc = sum_t (p_t vscale_t,g) a_tc + sum_t p_t vmin_t,g
//
// Codes enter an MFMA (v_mfma_f32_16x16x32_f16) as exact fp16 values 4 + code
// (one shift + one AND-OR per two codes); the per-page scale is folded into
// the other operand, which is split into two fp16 limbs (hi + lo represent
// the fp32 product of two fp16 numbers exactly), placed in different MFMA
// columns and summed after the product.  The +4 code offset and the minimum
// terms are per-page constants added on the VALU.
//
// One wave = one (sequence, KV head, group of <= 4 query heads, split of
// pages).  Lane l: column n = l & 15, row group w = l >> 4.  QK^T is computed
// transposed (rows = 16 tokens, columns = query head x limb), so each lane
// ends up holding the logits of tokens tau(w, 0..7) for head n & 3, which is
// exactly the K-slice it must feed to the PV MFMA: softmax needs no data
// movement besides the row-group max.  Online softmax runs in the log2
// domain; each split writes (m, l, O) and a second kernel merges the splits.
#include "kitty_internal.h"

namespace kitty {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float h2f(_Float16 h) { return (float)h; }

// Two fp16 MFMA operands 4 + code from one code word (combo 0 = A, 1 = B).
template <int COMBO>
__device__ __forceinline__ half8 unpack_codes(uint32_t word) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int sh = 8 - (2 * d + 8 * COMBO);
    const uint32_t x = sh >= 0 ? (word << sh) : (word >> (-sh));
    r[d] = (x & 0x03000300u) | 0x44004400u;
  }
  return __builtin_bit_cast(half8, r);
}

__device__ __forceinline__ floatx4 mfma(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

// hi / lo fp16 limbs of x; `limb` selects which one this lane supplies
__device__ __forceinline__ _Float16 limb_of(float x, int limb) {
  const _Float16 hi = (_Float16)x;
  const _Float16 lo = (_Float16)(x - (float)hi);
  return limb == 0 ? hi : (limb == 1 ? lo : (_Float16)0.0f);
}

struct SoftmaxState {
  float m;        // running max (log2 domain), -inf before the first token
  float l;        // this lane's share of the running denominator
  floatx4 o[8];   // PV accumulators: 8 blocks of 16 channels
  float corr[4];  // per value group: sum_t p_t (vmin - 4 vscale)
};

// Online-softmax update with 8 new logits (log2 domain, already scaled).
__device__ __forceinline__ void softmax_update(SoftmaxState& st, const float (&s)[8], float (&p)[8]) {
  float mp = s[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mp = fmaxf(mp, s[j]);
  mp = fmaxf(mp, __shfl_xor(mp, 16));
  mp = fmaxf(mp, __shfl_xor(mp, 32));
  const float mn = fmaxf(st.m, mp);
  const float alpha = exp2f(st.m - mn);
  float ps = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) { p[j] = exp2f(s[j] - mn); ps += p[j]; }
  st.l = st.l * alpha + ps;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.o[mb] *= alpha;
#pragma unroll
  for (int g = 0; g < 4; ++g) st.corr[g] *= alpha;
  st.m = mn;
}

template <int NHI>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  __shared__ float qs[4][kHeadDim];
  constexpr int NB = (NHI + 31) / 32;  // boost slot blocks
  constexpr int NF = NHI / 32;         // full ones
  const int split = blockIdx.x;
  const int hk = blockIdx.y / p.n_head_groups, hg = blockIdx.y % p.n_head_groups;
  const int b = blockIdx.z;
  const int lane = threadIdx.x, n = lane & 15, w = lane >> 4, hl = n & 3, limb = n >> 2;
  const int hq0 = hk * p.group + 4 * hg;
  const int gcount = min(4, p.group - 4 * hg);
  const bool col_ok = (limb < 2) && (hl < gcount);

  // queries of this head group -> LDS (fp32), zero for absent heads
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float q0 = 0.0f, q1 = 0.0f;
    if (h < gcount) {
      const _Float16* qp = p.q + ((size_t)b * p.n_q_heads + hq0 + h) * kHeadDim + 2 * lane;
      q0 = h2f(qp[0]);
      q1 = h2f(qp[1]);
    }
    qs[h][2 * lane] = q0;
    qs[h][2 * lane + 1] = q1;
  }
  __syncthreads();
  float qv[32];  // q of head hl at channels 32kb + 8w + j, zero unless col_ok
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[kb * 8 + j] = col_ok ? qs[hl][32 * kb + 8 * w + j] : 0.0f;

  int seq = p.seq_lens[b];
  seq = seq < 0 ? 0 : (seq > p.max_seq_len ? p.max_seq_len : seq);
  int P = seq / kPageTokens;
  const int ntail = seq - P * kPageTokens;
  if (P > p.max_pages) P = p.max_pages;
  const int p0 = split * p.pages_per_split;
  const int p1 = min(p0 + p.pages_per_split, P);
  const int tail_split = min(P / p.pages_per_split, p.n_split - 1);
  const bool do_tail = ntail > 0 && split == tail_split;

  const float sl2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;
  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) st.o[mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < 4; ++g) st.corr[g] = 0.0f;

  const int rb = rec_bytes(NHI);
  for (int pg = p0; pg < p1; ++pg) {
    const int phys = p.block_table[(size_t)b * p.max_pages + pg];
    if (phys < 0 || (int64_t)phys >= p.n_pages) continue;
    const uint8_t* rec = p.pages + (int64_t)phys * p.page_bytes + (int64_t)hk * rb;

    const u32x4 kw = *reinterpret_cast<const u32x4*>(rec + 16 * lane);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(rec + off_v(NHI) + 16 * lane);
    uint32_t bw[NB > 0 ? NB : 1];
#pragma unroll
    for (int bb = 0; bb < NF; ++bb) bw[bb] = *reinterpret_cast<const uint32_t*>(rec + off_kboost() + 4 * (lane * NF + bb));
    if (NB > NF) bw[NF] = lane < 32 ? *reinterpret_cast<const uint32_t*>(rec + off_kboost() + 256 * NF + 4 * lane) : 0u;
    half8 ksv[4], kmv[4], vsv[4], vmv[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      ksv[kb] = *reinterpret_cast<const half8*>(rec + off_kscale(NHI) + 2 * (32 * kb + 8 * w));
      kmv[kb] = *reinterpret_cast<const half8*>(rec + off_kmin(NHI) + 2 * (32 * kb + 8 * w));
      vsv[kb] = *reinterpret_cast<const half8*>(rec + off_vscale(NHI) + 2 * (32 * kb + 8 * w));
      vmv[kb] = *reinterpret_cast<const half8*>(rec + off_vmin(NHI) + 2 * (32 * kb + 8 * w));
    }

    // QK operand: limbs of q * kscale; constant part of the logits
    half8 bq[4];
    float cpart = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float prod = qv[kb * 8 + j] * h2f(ksv[kb][j]);
        const _Float16 val = limb_of(prod, limb);
        bq[kb][j] = val;
        cpart += (limb == 0 ? qv[kb * 8 + j] * h2f(kmv[kb][j]) : 0.0f) - 4.0f * (float)val;
      }
    half8 bb_op[NB > 0 ? NB : 1];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int s0 = 32 * bb + 8 * w;
      u32x2 ib = {0u, 0u};
      if (s0 < NHI) ib = *reinterpret_cast<const u32x2*>(rec + off_idx(NHI) + s0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        _Float16 val = (_Float16)0.0f;
        if (s0 + j < NHI) {
          const int ch = (int)((ib[j >> 2] >> (8 * (j & 3))) & 0x7Fu);  // channel < 128
          const float ksc = h2f(*reinterpret_cast<const _Float16*>(rec + off_kscale(NHI) + 2 * ch));
          const float prod = (col_ok ? qs[hl][ch] : 0.0f) * ksc * 0.25f;
          val = limb_of(prod, limb);
        }
        bb_op[bb][j] = val;
        cpart -= 4.0f * (float)val;
      }
    }

    floatx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      acc0 = mfma(unpack_codes<0>(kw[kb]), bq[kb], acc0);
      acc1 = mfma(unpack_codes<1>(kw[kb]), bq[kb], acc1);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      acc0 = mfma(unpack_codes<0>(bw[bb]), bb_op[bb], acc0);
      acc1 = mfma(unpack_codes<1>(bw[bb]), bb_op[bb], acc1);
    }
    float c = xor_sum(cpart, 4);
    c = xor_sum(c, 16);
    c = xor_sum(c, 32);
    float s[8], pr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (xor_sum(acc0[i], 4) + c) * sl2;
      s[4 + i] = (xor_sum(acc1[i], 4) + c) * sl2;
    }
    softmax_update(st, s, pr);

    // PV: operand limbs of p * vscale per value group, two 16-channel blocks each
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      half8 bp;
      float cg = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float vsc = h2f(vsv[g][j]);
        bp[j] = col_ok ? limb_of(pr[j] * vsc, limb) : (_Float16)0.0f;
        cg += pr[j] * (h2f(vmv[g][j]) - 4.0f * vsc);
      }
      st.corr[g] += cg;
      st.o[2 * g] = mfma(unpack_codes<0>(vw[g]), bp, st.o[2 * g]);
      st.o[2 * g + 1] = mfma(unpack_codes<1>(vw[g]), bp, st.o[2 * g + 1]);
    }
  }

  if (do_tail) {
    // fp16 tail tokens 32P .. seq-1: same contraction with fp16 K/V values
    const size_t toff = ((size_t)b * p.n_kv_heads + hk) * kPageTokens * kHeadDim;
    const _Float16* tk = p.tail_k + toff;
    const _Float16* tv = p.tail_v + toff;
    floatx4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      half8 bq;
#pragma unroll
      for (int j = 0; j < 8; ++j) bq[j] = limb == 0 ? (_Float16)qv[kb * 8 + j] : (_Float16)0.0f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = 16 * tb + n;
        half8 a = {};
        if (t < ntail) a = *reinterpret_cast<const half8*>(tk + (size_t)t * kHeadDim + 32 * kb + 8 * w);
        acc[tb] = mfma(a, bq, acc[tb]);
      }
    }
    float s[8], pr[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tb + 4 * w + i;
        const float v = xor_sum(acc[tb][i], 4) * sl2;
        s[4 * tb + i] = t < ntail ? v : -INFINITY;
      }
    softmax_update(st, s, pr);
    half8 bp;
#pragma unroll
    for (int j = 0; j < 8; ++j) bp[j] = col_ok ? limb_of(pr[j], limb) : (_Float16)0.0f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      half8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = j < 4 ? 4 * w + j : 16 + 4 * w + (j - 4);
        a[j] = t < ntail ? tv[(size_t)t * kHeadDim + 16 * mb + n] : (_Float16)0.0f;
      }
      st.o[mb] = mfma(a, bp, st.o[mb]);
    }
  }

  // merge lanes: hi + lo columns, row groups; write this split's partial
  float l = xor_sum(st.l, 16);
  l = xor_sum(l, 32);
  float cg[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    cg[g] = xor_sum(st.corr[g], 16);
    cg[g] = xor_sum(cg[g], 32);
  }
  float* dst = p.partial + (((size_t)b * p.n_q_heads + hq0 + hl) * p.n_split + split) * kPartialStride;
  const bool writer = (limb == 0) && (hl < gcount);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = xor_sum(st.o[mb][i], 4) + cg[mb >> 1];
      if (writer) dst[2 + 16 * mb + 4 * w + i] = o;
    }
  if (writer && w == 0) {
    dst[0] = st.m;
    dst[1] = l;
  }
}

// grid (batch * Hq), 128 threads: log-sum-exp merge of the splits
__global__ __launch_bounds__(128) void combine_kernel(DecodeParams p) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const float* src = p.partial + (size_t)bh * p.n_split * kPartialStride;
  float M = -INFINITY;
  for (int s = 0; s < p.n_split; ++s) M = fmaxf(M, src[s * kPartialStride]);
  float o = 0.0f;
  if (M != -INFINITY) {
    float L = 0.0f, acc = 0.0f;
    for (int s = 0; s < p.n_split; ++s) {
      const float* ps = src + s * kPartialStride;
      const float f = exp2f(ps[0] - M);
      L += f * ps[1];
      acc += f * ps[2 + c];
    }
    o = acc / L;
  }
  p.out[(size_t)bh * kHeadDim + c] = o;
}

template <int NHI>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.n_split, p.n_kv_heads * p.n_head_groups, p.batch);
  hipLaunchKernelGGL(decode_split_kernel<NHI>, grid, dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(p.batch * p.n_q_heads), dim3(kHeadDim), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

SplitPlan plan_splits(int batch, int n_kv_heads, int n_head_groups, int max_seq_len) {
  const int P = max_seq_len / kPageTokens;
  const long units = (long)batch * n_kv_heads * n_head_groups;
  const long target = 2048;  // waves: several per CU on 256 CUs
  long ns = (target + units - 1) / units;
  const long cap = P > 1 ? P : 1;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  int pps = (int)((P + ns - 1) / ns);
  if (pps < 1) pps = 1;
  int n_split = (P + pps - 1) / pps;
  if (n_split < 1) n_split = 1;
  return SplitPlan{n_split, pps};
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.n_hi) {
    case 0: return launch_decode_t<0>(p, stream);
    case 16: return launch_decode_t<16>(p, stream);
    case 32: return launch_decode_t<32>(p, stream);
    case 48: return launch_decode_t<48>(p, stream);
    case 64: return launch_decode_t<64>(p, stream);
    case 80: return launch_decode_t<80>(p, stream);
    case 96: return launch_decode_t<96>(p, stream);
    case 112: return launch_decode_t<112>(p, stream);
    case 128: return launch_decode_t<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kitty
