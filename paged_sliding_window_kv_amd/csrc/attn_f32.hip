// Paged attention in fp32 (small fp32 streams).
//
// Same operation as the bf16 kernel: O = softmax(s * Q K^T) V over the tokens
// of a sequence's page-table entries, no mask ("LingBot-Map Paged KV Cache",
// section 2), with an online softmax over 64-key tiles.  fp32 inputs,
// products and accumulation on the vector ALUs.
//
// One wave per workgroup; each lane owns one query row (Q and the output
// accumulator in registers).  A 64-key tile of K ([key][dim]) and V^T
// ([dim][key], the pool layout) is staged in LDS; every lane reads the same
// address at each step, so LDS reads are broadcasts.  Keys are processed in
// blocks of 16 with one rescale of the accumulator per block.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

constexpr int D = kHeadDim;
constexpr int KT = kKeyTile;
constexpr int ROWS = 64;
constexpr int KB = 16;

template <class Src>
__global__ __launch_bounds__(64) void attn_f32_kernel(const Src src) {
  const AttnParams& p = attn_base(src);
  __shared__ __attribute__((aligned(16))) float lk[KT * D];
  __shared__ __attribute__((aligned(16))) float lv[D * KT];

  const int L = blockIdx.x;
  const int g = L % p.groups_padded;
  const int qt = L / p.groups_padded;
  if (g >= p.groups) return;
  const int split = g % p.num_splits;
  const int sh = g / p.num_splits;
  const int h = sh % p.num_heads;
  const int seq = sh / p.num_heads;
  int q0, qn, ebase, ecount;
  attn_seq(src, seq, q0, qn, ebase, ecount);
  const int row0 = qt * ROWS;
  if (row0 >= qn) return;
  const int per = (ecount + p.num_splits - 1) / p.num_splits;
  const int eb = ebase + min(ecount, split * per);
  const int ee = ebase + min(ecount, (split + 1) * per);

  const int H = p.num_heads;
  const int P = p.page_size;
  const int lane = threadIdx.x;
  const int qrow = row0 + lane;
  const bool qvalid = qrow < qn;
  const float* qg = static_cast<const float*>(p.q);
  const float* kg = static_cast<const float*>(p.k_pool);
  const float* vg = static_cast<const float*>(p.v_pool);

  float q[D], o[D];
  {
    const float* qp = qg + (static_cast<size_t>(q0 + (qvalid ? qrow : 0)) * H + h) * D;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
      const float4 v = qvalid ? *reinterpret_cast<const float4*>(qp + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = v.x;
      q[i + 1] = v.y;
      q[i + 2] = v.z;
      q[i + 3] = v.w;
    }
  }
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int e = eb; e < ee; ++e) {
    int pid, len;
    attn_entry(src, e, pid, len);
    for (int kt = 0; kt * KT < len; ++kt) {
      const int nk = min(KT, len - kt * KT);
      __syncthreads();
      const float* kb = kg + ((static_cast<size_t>(pid) * H + h) * P + kt * KT) * D;
      const float* vb = vg + (static_cast<size_t>(pid) * H + h) * D * P + kt * KT;
      for (int c = lane; c < KT * D / 4; c += 64) {
        reinterpret_cast<float4*>(lk)[c] = reinterpret_cast<const float4*>(kb)[c];
        // pool elements 4c'..4c'+3 of a V^T row hold slots v_slot_pos(4c')..+3
        const int dd = c / (KT / 4), p4 = (c % (KT / 4)) * 4;
        const int k4 = v_slot_pos(p4);
        float4 v = *reinterpret_cast<const float4*>(vb + static_cast<size_t>(dd) * P + p4);
        if (k4 + 0 >= nk) v.x = 0.f;
        if (k4 + 1 >= nk) v.y = 0.f;
        if (k4 + 2 >= nk) v.z = 0.f;
        if (k4 + 3 >= nk) v.w = 0.f;
        *reinterpret_cast<float4*>(lv + dd * KT + k4) = v;
      }
      __syncthreads();
      for (int j0 = 0; j0 < nk; j0 += KB) {
        float s[KB];
        float bm = -INFINITY;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const float* kr = lk + (j0 + j) * D;
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < D; i += 4) {
            const float4 kv = *reinterpret_cast<const float4*>(kr + i);
            acc = __builtin_fmaf(q[i], kv.x, acc);
            acc = __builtin_fmaf(q[i + 1], kv.y, acc);
            acc = __builtin_fmaf(q[i + 2], kv.z, acc);
            acc = __builtin_fmaf(q[i + 3], kv.w, acc);
          }
          s[j] = (j0 + j < nk) ? acc * p.scale_log2 : -INFINITY;
          bm = fmaxf(bm, s[j]);
        }
        const float m_new = fmaxf(m_run, bm);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          s[j] = __builtin_amdgcn_exp2f(s[j] - m_new);
          rs += s[j];
        }
        l_run = __builtin_fmaf(l_run, alpha, rs);
#pragma unroll
        for (int i = 0; i < D; ++i) {
          float acc = o[i] * alpha;
          const float* vr = lv + i * KT + j0;
#pragma unroll
          for (int j = 0; j < KB; j += 4) {
            const float4 vv = *reinterpret_cast<const float4*>(vr + j);
            acc = __builtin_fmaf(s[j], vv.x, acc);
            acc = __builtin_fmaf(s[j + 1], vv.y, acc);
            acc = __builtin_fmaf(s[j + 2], vv.z, acc);
            acc = __builtin_fmaf(s[j + 3], vv.w, acc);
          }
          o[i] = acc;
        }
      }
    }
  }

  if (!qvalid) return;
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse_nat = empty ? -INFINITY : (m_run + log2f(l_run)) * 0.69314718055994530942f;
  const size_t orow = static_cast<size_t>(q0 + qrow) * H + h;
  float* out = p.num_splits == 1 ? static_cast<float*>(p.o) + orow * D
                                 : p.part_o + (static_cast<size_t>(split) * p.total_q * H + orow) * D;
#pragma unroll
  for (int i = 0; i < D; i += 4)
    *reinterpret_cast<float4*>(out + i) = make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
  if (p.num_splits == 1) {
    if (p.lse) p.lse[orow] = lse_nat;
  } else {
    p.part_lse[static_cast<size_t>(split) * p.total_q * H + orow] = lse_nat;
  }
}

}  // namespace

int attn_f32_rows_per_tile() { return ROWS; }

template <class Src>
static hipError_t launch_impl(const Src& src, hipStream_t stream) {
  const AttnParams& p = attn_base(src);
  const dim3 grid(static_cast<unsigned>(p.q_tiles) * p.groups_padded);
  hipLaunchKernelGGL((attn_f32_kernel<Src>), grid, dim3(64), 0, stream, src);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) { return launch_impl(p, stream); }
hipError_t launch_attn_f32(const AttnParamsInline& p, hipStream_t stream) { return launch_impl(p, stream); }

}  // namespace kvc
