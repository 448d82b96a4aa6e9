// Paged attention, bf16 inputs, fp32 accumulation, for CDNA4 (gfx950).
//
// Computes O = softmax(s * Q K^T) V for each query sequence and head over the
// tokens of the sequence's page-table entries, with no mask: the visible
// table already lists exactly the tokens a frame or chunk attends to, and
// each page carries its valid length ("LingBot-Map Paged KV Cache", section
// 2; "vLLM-Omni RFC #2727", section 1: global attention over the window).
// The online softmax processes one 64-key tile at a time and keeps a running
// maximum and sum per query, so no score matrix is stored.
//
// Mapping to the hardware
//  * One workgroup = 2*NB waves covering NB*32 query rows of one (sequence,
//    head, key split).  Waves w and w+NB own the same 32 rows: each 128-key
//    step (two 64-key tiles per barrier) gives the first tile to wave w and
//    the second to wave w+NB, each with its own online-softmax state; the
//    two states are merged through LDS at the end.  With NB = 8 that is 16
//    waves, four per SIMD, so one wave's products can run under another's
//    softmax arithmetic.  The tile's queries sit in LDS (loaded by direct
//    loads with the first key tiles); Q fragments are re-read there every
//    step rather than held in registers.
//  * Variant NB = 8 + extra block covers 272 rows (the 262 queries of a
//    frame fit one workgroup): the 16-row extra block runs on
//    v_mfma_f32_16x16x32_bf16, waves 0..3 (one per SIMD) each taking one
//    32-key quarter of every step; its accumulators wait in LDS between
//    steps, and the four quarter states are merged at the end.
//  * The online softmax forms each tile's probabilities against the running
//    maximum as it stands and accepts them when the lane's sum is bounded
//    (see kSumBound); the tile maximum is taken only on a wave's first tile
//    and in the rare case a sum exceeds the bound.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims, B = 16 dims x 32
//    queries, both from LDS.  In the 32x32 accumulator each lane then
//    holds 16 scores of a single query, so the row maximum and row sum are
//    in-lane reductions (shallow trees) plus one v_permlane32_swap between
//    lane l and lane l + 32.
//  * The probabilities are reused in registers as the B operand of
//    O^T = V^T P^T (A = 32 dims x 16 keys of V^T from LDS).  Which k-slot of
//    the instruction carries which key is free (k is summed over), so the
//    key order of the accumulator layout is used as is: half-wave h supplies
//    keys {4h..4h+3, 8+4h..8+4h+3} of each 16-key group.  The V pool stores
//    every 16-slot group of a V^T row in exactly that order (middle two
//    4-slot groups swapped), so a 16-byte chunk of pool memory is one MFMA
//    operand fragment.
//  * K and V^T tiles (8 KiB each) stream through a 6-stage LDS ring filled
//    by direct global->LDS loads (global_load_lds_dwordx4): up to four tiles
//    are in flight per workgroup while a pair is consumed, without staging
//    registers.  Each wave waits only for its own loads of the tile about to
//    be used (s_waitcnt vmcnt(n)) before the workgroup barrier.  16-byte
//    chunks are XOR-swizzled by row (the swizzle is applied through the
//    global addresses each lane fetches) so that fragment reads spread over
//    all LDS banks.
//  * Keys past a page's valid length: scores are set to -inf, and the V^T
//    slots of those keys are zeroed in LDS before use, so stale pool
//    contents (even NaN) never reach O.
//  * The 1-D grid is ordered so that all query tiles of one (sequence, head,
//    split) share the same index modulo 8 and therefore the same XCD (and its
//    L2), which serves their repeated reads of that head's K/V.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.hpp"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float floatx8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef _Float16 halfx4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = kHeadDim;         // 64
constexpr int KT = kKeyTile;        // 64 keys per tile
constexpr int TILE_ELEMS = KT * D;  // 4096 bf16 = 8 KiB per tensor
constexpr int STAGES = 6;           // LDS ring depth in 64-key tiles (96 KiB)
constexpr int DMA_PER_TILE = 16;    // 1 KiB global->LDS loads per tile (8 for K, 8 for V)

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with expcnt and lgkmcnt left
// open, and lgkmcnt(0) with the others left open.
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkmcnt0 = 0xC07F;
// A tile's probabilities are formed against the running maximum m as it
// stands (no maximum of the tile is taken on the way).  They are accepted when
// every lane's sum of them is at most kSumBound, which bounds each one; only
// otherwise (a row whose scores outgrow m by several units, or m not yet set)
// is the tile's maximum taken, O and the row sum rescaled, and the
// probabilities formed again.  Values up to kSumBound are far from fp32 or
// bf16 overflow, and the final division by the row sum is exact whichever
// reference was used.
constexpr float kSumBound = 65536.f;  // 2^16

// 16-byte chunk c of LDS row r is stored at physical chunk c ^ swz(r).  Rows
// are 128 bytes, so 16 consecutive rows read at the same logical chunk cover
// all 64 banks exactly once, and any 8 consecutive rows cover 32 banks once.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(base + row * D + ((chunk ^ swz(row)) << 3));
}

__device__ __forceinline__ bf16x8 to_bf16x8(floatx16 s, int base) {
  floatx8 f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = s[base + j];
  return __builtin_convertvector(f, bf16x8);
}

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float floatx2 __attribute__((__vector_size__(2 * sizeof(float))));

// One v_cvt_pk_bf16_f32 (round to nearest even); cat4 assembles four pairs
// into one operand fragment (element 2q+i of the result is element i of pair q).
__device__ __forceinline__ bf16x2 cvt2(float a, float b) {
  const floatx2 f = {a, b};
  return __builtin_convertvector(f, bf16x2);
}
__device__ __forceinline__ bf16x8 cat4(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lanes l and l+32 hold the two halves of a query's keys; these combine the
// pair with one v_permlane32_swap (which hands each lane its partner's value)
// instead of an LDS permute.  With operands (x, y) the instruction returns
// r0[l] = x[l%32] for l < 32 and y[l%32] above, r1[l] = x[32 + l%32] for
// l < 32 and y[32 + l%32] above, so for y = x, {r0, r1} is {own, partner} in
// every lane.  (The elements are copied to scalars before reinterpreting
// them: a bit cast applied directly to an element of the returned vector
// reads element 0.)
__device__ __forceinline__ void pair_values(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_values(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_values(x, a, b);
  return a + b;
}

// Maximum and sum of the 32 scores a lane holds for one 64-key tile, as
// shallow trees (depth 4-5) rather than 32-long dependency chains.
__device__ __forceinline__ float tile_max(const floatx16& a, const floatx16& b) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fmaxf(fmaxf(fmaxf(a[i], a[i + 8]), b[i]), b[i + 8]);
  return fmaxf(fmaxf(fmaxf(c[0], c[1]), c[2]), fmaxf(fmaxf(fmaxf(c[3], c[4]), c[5]), fmaxf(c[6], c[7])));
}
__device__ __forceinline__ float tile_sum(const floatx16& a, const floatx16& b) {
  float u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = (a[i] + a[i + 8]) + (b[i] + b[i + 8]);
  return ((u[0] + u[1]) + (u[2] + u[3])) + ((u[4] + u[5]) + (u[6] + u[7]));
}
__device__ __forceinline__ float half_max(const floatx16& a) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fmaxf(fmaxf(a[i], a[i + 4]), fmaxf(a[i + 8], a[i + 12]));
  return fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
}
__device__ __forceinline__ float half_sum(const floatx16& a) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = (a[i] + a[i + 4]) + (a[i + 8] + a[i + 12]);
  return (c[0] + c[1]) + (c[2] + c[3]);
}

// Cursor over (table entry, 64-key tile of the page).
struct Cursor {
  int e, kt, len, pid;
};

template <class Src>
__device__ __forceinline__ void cursor_first(const Src& src, int eb, int ee, Cursor& c) {
  c.e = eb;
  c.kt = 0;
  c.len = 0;
  c.pid = 0;
  while (c.e < ee) {
    attn_entry(src, c.e, c.pid, c.len);
    if (c.len > 0) break;
    ++c.e;
  }
}

template <class Src>
__device__ __forceinline__ void cursor_next(const Src& src, int ee, Cursor& c) {
  if ((c.kt + 1) * KT < c.len) {
    ++c.kt;
    return;
  }
  c.kt = 0;
  ++c.e;
  while (c.e < ee) {
    attn_entry(src, c.e, c.pid, c.len);
    if (c.len > 0) break;
    ++c.e;
  }
}

// Lanes l, l^16, l^32 and l^48 hold the four 4-key groups of one query in the
// 16x16 layout of the extra block; v_permlane16_swap pairs l with l^16 the way
// v_permlane32_swap pairs l with l^32.
__device__ __forceinline__ void pair16_values(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float quad_max(float x) {
  float a, b;
  pair16_values(x, a, b);
  return pair_max(fmaxf(a, b));
}
__device__ __forceinline__ float quad_sum(float x) {
  float a, b;
  pair16_values(x, a, b);
  return pair_sum(a + b);
}

// KV8: the pools hold FP8 (OCP E4M3) codes with per-(token, head) int8 row
// exponents (layout in kvc.h).  The ring then stages the codes and exponents
// of each tile (8,320 bytes), and after each pair's barrier the workgroup
// converts the pair into two bf16 tiles with v_cvt_scalef32_pk_bf16_fp8
// applying 2^e; every later step is the bf16 kernel's.  The dequantised
// values are exactly bf16 numbers (3-bit mantissas times powers of two).
template <int NB, bool XB, class Src, bool KV8 = false>
__global__ __launch_bounds__(NB * 128) void attn_bf16_kernel(const Src src) {
  static_assert(!XB || NB >= 2, "the extra block is shared by waves 0..3");
  const AttnParams& p = attn_base(src);
  constexpr int W = 2 * NB;                             // waves: two per 32-row block
  constexpr int ROWS = NB * 32 + (XB ? 16 : 0);
  constexpr int LPT = (DMA_PER_TILE + W - 1) / W;       // direct loads per wave per tile
  constexpr int TILE_BYTES = 2 * TILE_ELEMS * 2;        // K and V^T of one bf16 tile
  constexpr int STAGE8 = 2 * TILE_ELEMS + 2 * KT;       // FP8 stage: K codes, V codes, K exps, V exps
  constexpr int RING_BYTES = KV8 ? 2 * TILE_BYTES + STAGES * STAGE8 : STAGES * TILE_BYTES;
  constexpr int Q_BYTES = ROWS * D * 2;
  // Extra block: each quarter wave's O^T accumulator [4][16][64] (fp32)
  // lives in LDS between steps, so it does not hold registers through the
  // main products.
  constexpr int XO_BYTES = XB ? 4 * 16 * 64 * 4 : 0;
  // End of the kernel: the odd-tile waves' states [NB][34][64] and the extra
  // block's quarter states [3][18][64] (fp32), over the idle ring.
  constexpr int MERGE_BYTES = (NB * 34 + (XB ? 3 * 18 : 0)) * 64 * 4;
  constexpr int SMEM = RING_BYTES + Q_BYTES + XO_BYTES > MERGE_BYTES ? RING_BYTES + Q_BYTES + XO_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  // bf16 tiles: the ring (STAGES tiles), or the converted pair (KV8)
  uint16_t* const lds_t = reinterpret_cast<uint16_t*>(smem);
  uint8_t* const lds8 = smem + (KV8 ? 2 * TILE_BYTES : 0);  // FP8 stages
  uint16_t* const lds_q = reinterpret_cast<uint16_t*>(smem + RING_BYTES);  // queries, swizzled rows
  floatx4* const lds_xo = reinterpret_cast<floatx4*>(smem + RING_BYTES + Q_BYTES);  // [wave][db][lane]

  // ---- which (sequence, head, split, query tile) ----------------------------
  int g, qt;
  attn_tile_of(p, blockIdx.x, g, qt);
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
  const float sl2 = p.scale_log2;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  // Block blk = wave mod NB; waves below NB take the first tile of every
  // 128-key step, the others the second.
  const bool odd = wave >= NB;
  const int blk = odd ? wave - NB : wave;
  const int wrow0 = row0 + blk * 32;
  const bool active = wrow0 < qn;
  // Extra block (XB): 16 rows NB*32 .. NB*32+15 of the tile, on 16x16x32
  // products; waves 0..3 each take one 32-key quarter of every 128-key step.
  const int xrow0 = row0 + NB * 32;
  const bool xblock = XB && xrow0 < qn;  // workgroup-uniform
  const bool xactive = xblock && wave < 4;
  const int c16 = lane & 15, g4 = lane >> 4;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k_pool);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v_pool);
  const size_t page_stride = static_cast<size_t>(H) * P * D;  // elements per page (K or V)
  const size_t head_off = static_cast<size_t>(h) * P * D;

  // ---- queries of the tile -> LDS ---------------------------------------------
  // Q fragments (B operand of S^T = K Q^T: Q[row][16*st + 8*lh .. +7]) are read
  // from here at every step rather than held in registers.  The rows come by
  // direct loads of 8 rows (1 KiB) each, issued before the first tiles so
  // that both latencies overlap; the tile waits below cover them (loads
  // complete in issue order), and the first ring barrier publishes lds_q and
  // lds_xo.  Rows past the sequence repeat its last row: their outputs are
  // never written.
  for (int j = wave; j < ROWS / 8; j += W) {
    const int r = j * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ swz(r);  // logical chunk held by physical chunk lane%8
    const int row = min(row0 + r, qn - 1);
    const uint16_t* gp = qg + (static_cast<size_t>(q0 + row) * H + h) * D + ch * 8;
    __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds_q + j * 512), 16, 0, 0);
  }
  if (XB && xactive) {
#pragma unroll
    for (int db = 0; db < 4; ++db) lds_xo[(wave * 4 + db) * 64 + lane] = floatx4{};
  }

  // ---- this wave's share of each tile's 16 direct loads -----------------------
  // Load `inst` of a tile fills 1 KiB = LDS positions 64*part .. 64*part+63 of
  // K (inst < 8) or V^T (inst >= 8); lane l fills position 64*part + l, i.e.
  // row 8*part + l/8, physical chunk l%8, which holds logical chunk
  // (l%8) ^ swz(row).  Surplus slots (16 not divisible by the wave count)
  // repeat the last load: identical bytes to identical addresses.
  int dma_goff[LPT], dma_loff[LPT];
  bool dma_v[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = min(wave * LPT + j, DMA_PER_TILE - 1);
    const int is_v = inst >> 3, part = inst & 7;
    const int row = part * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    dma_v[j] = is_v != 0;
    // K tile rows are keys ([slot][dim]); V^T tile rows are dims ([dim][slot]).
    dma_goff[j] = is_v ? row * P + chunk * 8 : row * D + chunk * 8;
    dma_loff[j] = is_v * TILE_ELEMS + part * 512;
  }
  // KV8 loads: inst 0-3 K codes (1 KiB each), 4-7 V codes, 8-11 K exponents
  // and 12-15 V exponents (16 bytes each, lane 0 only).  Stage bytes:
  // [0, 4096) K codes [slot][dim], [4096, 8192) V codes [slot][dim],
  // [8192, 8256) K exponents, [8256, 8320) V exponents.
  int dma8_kind[LPT], dma8_off[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = min(wave * LPT + j, DMA_PER_TILE - 1);
    const int kind = inst >> 2, q = inst & 3;
    dma8_kind[j] = kind;
    dma8_off[j] = kind < 2 ? kind * 4096 + q * 1024 : 8192 + (kind - 2) * KT + q * 16;
  }
  const uint8_t* __restrict__ kg8 = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* __restrict__ vg8 = static_cast<const uint8_t*>(p.v_pool);
  const size_t codes_bytes = static_cast<size_t>(p.num_pool_pages) * H * P * D;  // exponents follow
  auto issue = [&](const Cursor& c, int stage) {
    if constexpr (KV8) {
      const size_t row0 = (static_cast<size_t>(c.pid) * H + h) * P + c.kt * KT;  // first slot row of the tile
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int kind = dma8_kind[j];
        const uint8_t* base = (kind & 1) ? vg8 : kg8;
        if (kind < 2) {
          // (the source goes in as const void*: a byte pointer there leaves the
          // host side of this instantiation without its launch stub)
          const void* gp = base + row0 * D + (dma8_off[j] & 4095) + lane * 16;
          __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds8 + stage * STAGE8 + dma8_off[j]), 16, 0, 0);
        } else if (lane == 0) {
          const void* gp = base + codes_bytes + row0 + (dma8_off[j] - 8192 - (kind - 2) * KT);
          __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds8 + stage * STAGE8 + dma8_off[j]), 16, 0, 0);
        }
      }
    } else {
      const size_t base = static_cast<size_t>(c.pid) * page_stride + head_off;
      const int koff = c.kt * KT * D, voff = c.kt * KT;
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const uint16_t* gp = (dma_v[j] ? vg + voff : kg + koff) + base + dma_goff[j];
        __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds_t + stage * 2 * TILE_ELEMS + dma_loff[j]), 16, 0, 0);
      }
    }
  };
  // KV8: converts staged tile `stage` (nk valid keys) into bf16 buffer `b`:
  // K items (token, 8-dim chunk) become 16-byte row writes; V items (4
  // consecutive tokens, 2 dims) become one 8-byte write of 4 slots per dim
  // into its V^T row (the pool slot order keeps aligned runs of 4 slots
  // contiguous), with the chunk swizzle.  Keys past nk become zeros.
  auto convert = [&](int stage, int b, int nk) {
    const uint8_t* st8 = lds8 + stage * STAGE8;
    uint16_t* tk = lds_t + b * 2 * TILE_ELEMS;
    // The per-thread addresses below are recomputed at every call (a few
    // integer operations) rather than hoisted out of the key loop, where they
    // would hold registers the products need.
    int t0 = tid;
    asm volatile("" : "+v"(t0));
    typedef __bf16 bf16x2_ __attribute__((__vector_size__(2 * sizeof(__bf16))));
    for (int it = t0; it < 2 * KT * 8; it += W * 64) {
      if (it < KT * 8) {
        const int r = it >> 3, ch = it & 7;  // token, 8-dim chunk
        const uint2 w = *reinterpret_cast<const uint2*>(st8 + r * D + ch * 8);
        const int e = static_cast<int8_t>(st8[8192 + r]);
        const float sc = __builtin_ldexpf(1.f, e);
        bf16x2_ v2[4];
        v2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.x), sc, false);
        v2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.x), sc, true);
        v2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.y), sc, false);
        v2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.y), sc, true);
        uint32_t u[4];
        __builtin_memcpy(u, v2, sizeof u);
        if (r >= nk) u[0] = u[1] = u[2] = u[3] = 0u;
        *reinterpret_cast<uint4*>(tk + r * D + ((ch ^ swz(r)) << 3)) = make_uint4(u[0], u[1], u[2], u[3]);
      } else {
        const int q = it - KT * 8;
        const int r0 = (q >> 5) * 4, d0 = (q & 31) * 2;  // tokens r0..r0+3, dims d0, d0+1
        uint32_t v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = r0 + t;
          const int w = *reinterpret_cast<const uint16_t*>(st8 + 4096 + r * D + d0);
          const int e = static_cast<int8_t>(st8[8192 + KT + r]);
          const bf16x2_ c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, __builtin_ldexpf(1.f, e), false);
          __builtin_memcpy(&v[t], &c2, 4);
          if (r >= nk) v[t] = 0u;
        }
        const int pos = v_slot_pos(r0);  // slots r0..r0+3 sit at pos..pos+3
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = d0 + i;  // dim
          const int sh = 16 * i;
          const uint32_t lo = ((v[0] >> sh) & 0xFFFFu) | (((v[1] >> sh) & 0xFFFFu) << 16);
          const uint32_t hi = ((v[2] >> sh) & 0xFFFFu) | (((v[3] >> sh) & 0xFFFFu) << 16);
          *reinterpret_cast<uint2*>(tk + TILE_ELEMS + row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7))) =
              make_uint2(lo, hi);
        }
      }
    }
  };
  // Zero the V^T slots of keys nk..63 of a staged tile.  In a pool row, key k
  // of a 16-key group sits at element sigma(k) of the group (sigma swaps the
  // middle two 4-slot groups); the 16-byte chunk is then swizzled by row.
  auto zero_tail = [&](uint16_t* lv, int nk) {
    for (int it = tid; it < D * 16; it += W * 64) {
      const int row = it >> 4, grp = it & 15;  // 4-key group in key order
      const int k0 = grp * 4;
      if (k0 + 4 <= nk) continue;
      const int sg = (grp & ~3) | ((grp & 1) << 1) | ((grp >> 1) & 1);
      const int pos = sg * 4;
      uint16_t* rp = lv + row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k0 + e >= nk) rp[e] = 0;
    }
  };

  float m_run = -INFINITY;  // running max of scaled scores (log2 domain)
  bool mset = false;        // m_run set (wave-uniform)
  float l_run = 0.f;        // this lane's partial row sum
  floatx16 o0 = {}, o1 = {};
  float xm = -INFINITY, xl = 0.f;  // extra block: this wave's key quarters
  bool xset = false;

  // Tiles are consumed two at a time (128 keys per barrier).  Tile t lives in
  // ring stage t % STAGES; up to STAGES - 2 tiles beyond the current pair are
  // in flight.
  Cursor cc, lc;
  cursor_first(src, eb, ee, cc);
  lc = cc;
  int ni = 0, nc = 0;  // tiles issued, tiles consumed
  for (int s = 0; s < STAGES - 2 && lc.e < ee; ++s) {
    issue(lc, ni % STAGES);
    cursor_next(src, ee, lc);
    ++ni;
  }
  while (nc < ni) {
    const bool two = ni >= nc + 2;
    const int outstanding = ni - nc - (two ? 2 : 1);
    if (outstanding >= 2)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LPT));
    else if (outstanding == 1)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(LPT));
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __builtin_amdgcn_s_barrier();
    // The previous pair's stages are free now; they are refilled after this
    // pair's products (below), so that the waves do not all queue their loads
    // on the vector-memory pipe at the same moment.
    Cursor cb = cc;
    const int nka = min(KT, cc.len - cc.kt * KT);
    int nkb = 0;
    if (two) {
      cursor_next(src, ee, cb);
      nkb = min(KT, cb.len - cb.kt * KT);
    }
    const int sa = KV8 ? 0 : nc % STAGES, sb = KV8 ? 1 : (nc + 1) % STAGES;
    uint16_t* const lka = lds_t + sa * 2 * TILE_ELEMS;
    uint16_t* const lva = lka + TILE_ELEMS;
    uint16_t* const lkb = lds_t + sb * 2 * TILE_ELEMS;
    uint16_t* const lvb = lkb + TILE_ELEMS;
    if constexpr (KV8) {
      // Everyone is done with the previous pair's bf16 tiles (barrier above).
      convert(nc % STAGES, 0, nka);
      if (two) convert((nc + 1) % STAGES, 1, nkb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
      __builtin_amdgcn_s_barrier();
    } else if (nka < KT || (two && nkb < KT)) {
      if (nka < KT) zero_tail(lva, nka);
      if (two && nkb < KT) zero_tail(lvb, nkb);
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
      __builtin_amdgcn_s_barrier();
    }

    const int nk = odd ? nkb : nka;  // this wave's tile (nkb = 0 without a second tile)
    if (active && nk > 0) {
      const uint16_t* lk = odd ? lkb : lka;
      const uint16_t* lv = odd ? lvb : lva;
      // Scores of the tile (keys 0..31 then 32..63, four K fragments live at
      // a time: four reads, then their four products), keys past nk set to
      // -inf.
      auto scores = [&](floatx16& s0, floatx16& s1) {
        bf16x8 qf[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) qf[st] = lds_frag(lds_q, blk * 32 + lr, 2 * st + lh);
        s0 = floatx16{};
        s1 = floatx16{};
        __builtin_amdgcn_s_setprio(1);
        {
          bf16x8 kf[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) kf[st] = lds_frag(lk, lr, 2 * st + lh);
#pragma unroll
          for (int st = 0; st < 4; ++st) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s0, 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x8, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          bf16x8 kf[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) kf[st] = lds_frag(lk, 32 + lr, 2 * st + lh);
#pragma unroll
          for (int st = 0; st < 4; ++st) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s1, 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x8, 4, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (nk < KT) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
            if (key >= nk) s0[r] = -INFINITY;
            if (key + 32 >= nk) s1[r] = -INFINITY;
          }
        }
      };
      // Probabilities against the running maximum, in place; returns this
      // lane's sum of them.
      auto probs = [&](floatx16& s0, floatx16& s1) {
        const float nm = -m_run;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, nm));
          s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, nm));
        }
        return tile_sum(s0, s1);
      };
      floatx16 s0, s1;
      scores(s0, s1);
      if (!mset) {  // this wave's first tile: start from its exact maximum
        m_run = pair_max(tile_max(s0, s1)) * sl2;
        mset = true;
      }
      float lt = probs(s0, s1);
      if (__any(!(lt <= kSumBound))) {
        // Rare: take the tile's maximum (from the scores formed again: the K
        // tile is still in LDS) and rescale.
        scores(s0, s1);
        const float mx = pair_max(tile_max(s0, s1)) * sl2;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          o0[r] *= alpha;
          o1[r] *= alpha;
        }
        lt = probs(s0, s1);
      }
      l_run += lt;
      // V fragments are read only now: reading them during the softmax would
      // keep K, V and the scores live together (other waves hide the wait).
      // Each half of O^T takes four reads, then its four products.
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) pb[t] = to_bf16x8(t < 2 ? s0 : s1, 8 * (t & 1));
      {
        bf16x8 vf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) vf[t] = lds_frag(lv, lr, 2 * t + lh);
#pragma unroll
        for (int t = 0; t < 4; ++t) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pb[t], o0, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x8, 4, 0);
      }
      {
        bf16x8 vf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) vf[t] = lds_frag(lv, 32 + lr, 2 * t + lh);
#pragma unroll
        for (int t = 0; t < 4; ++t) o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pb[t], o1, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x8, 4, 0);
      }
    }

    if (XB && xactive) {
      // Extra block: this wave's 32-key quarter kq..kq+31 of the step, as two
      // 16-key blocks of S^T (16 keys x 16 queries, v_mfma_f32_16x16x32_bf16).
      // Block c holds keys kq + 8c + {0..7, 16..23}, so that the 4-key groups
      // lane group g4 receives are exactly the two halves of V^T chunk
      // kq/8 + g4 (pool slot order) and P feeds O^T = V^T P^T unchanged.
      const int tile = wave >> 1, kq = 32 * (wave & 1);
      const int nkt = tile ? nkb : nka;
      if (nkt > kq) {
        const uint16_t* lk = tile ? lkb : lka;
        const uint16_t* lv = tile ? lvb : lva;
        const int kr = kq + (c16 & 7) + 16 * (c16 >> 3);
        auto xscores = [&](floatx4& sa0, floatx4& sa1) {
          sa0 = floatx4{};
          sa1 = floatx4{};
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ds = 0; ds < 2; ++ds) {
            const bf16x8 qx = lds_frag(lds_q, NB * 32 + c16, 4 * ds + g4);
            sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(lk, kr, 4 * ds + g4), qx, sa0, 0, 0, 0);
            sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(lk, kr + 8, 4 * ds + g4), qx, sa1, 0, 0, 0);
          }
          __builtin_amdgcn_s_setprio(0);
          if (nkt < kq + 32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int idx = 4 * g4 + i;
              const int key = kq + (idx & 7) + 16 * (idx >> 3);
              if (key >= nkt) sa0[i] = -INFINITY;
              if (key + 8 >= nkt) sa1[i] = -INFINITY;
            }
          }
        };
        auto xmax = [&](const floatx4& sa0, const floatx4& sa1) {
          return quad_max(fmaxf(fmaxf(fmaxf(sa0[0], sa0[1]), fmaxf(sa0[2], sa0[3])),
                                fmaxf(fmaxf(sa1[0], sa1[1]), fmaxf(sa1[2], sa1[3])))) * sl2;
        };
        floatx8 pf;
        auto xprobs = [&](const floatx4& sa0, const floatx4& sa1) {
          const float nm = -xm;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa0[i], sl2, nm));
            pf[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa1[i], sl2, nm));
          }
          return ((pf[0] + pf[1]) + (pf[2] + pf[3])) + ((pf[4] + pf[5]) + (pf[6] + pf[7]));
        };
        floatx4 sa0, sa1;
        xscores(sa0, sa1);
        if (!xset) {
          xm = xmax(sa0, sa1);
          xset = true;
        }
        float xlt = xprobs(sa0, sa1);
        floatx4 xo[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) xo[db] = lds_xo[(wave * 4 + db) * 64 + lane];
        if (__any(!(xlt <= kSumBound))) {
          xscores(sa0, sa1);
          const float m_new = fmaxf(xm, xmax(sa0, sa1));
          const float alpha = xm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(xm - m_new);
          xm = m_new;
          xl *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) xo[db] *= alpha;
          xlt = xprobs(sa0, sa1);
        }
        xl += xlt;
        const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          xo[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(lv, db * 16 + c16, kq / 8 + g4), pb, xo[db], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) lds_xo[(wave * 4 + db) * 64 + lane] = xo[db];
      }
    }
    for (int s = 0; s < 2 && lc.e < ee; ++s) {
      issue(lc, ni % STAGES);
      cursor_next(src, ee, lc);
      ++ni;
    }
    nc += two ? 2 : 1;
    if (two) cc = cb;
    cursor_next(src, ee, cc);
  }

  // ---- epilogue ---------------------------------------------------------------
  // Writes one row's result: normalised O (bf16) and lse, or the split's
  // partial O and lse.  `get(j)` returns the unnormalised O of dims
  // d0[j/4] + j%4 (4 dims per run, `runs` runs); m is the maximum, ltot the
  // row sum; the lse is written by lanes with `lse_lane`.  A partial O goes
  // out in fp16 as O * 2^-E, E the smallest non-negative integer that keeps
  // the row's largest magnitude within 2^15 (0 for any ordinary row), with
  // 2^E beside it; `row_max` combines a lane's maximum with those of the
  // other lanes holding the same row (which share the row's validity).
  auto write_row = [&](int row, auto get, const int* d0, auto runs_c, float m, float ltot, bool lse_lane,
                       auto row_max) {
    constexpr int runs = decltype(runs_c)::value;
    const bool empty = !(ltot > 0.f);
    const float inv = empty ? 0.f : 1.f / ltot;
    const float lse_nat = empty ? -INFINITY : (m + __log2f(ltot)) * 0.69314718055994530942f;
    const size_t orow = static_cast<size_t>(q0 + row) * H + h;
    if (p.num_splits == 1) {
      uint16_t* og = static_cast<uint16_t*>(p.o) + orow * D;
#pragma unroll
      for (int r4 = 0; r4 < runs; ++r4) {
        floatx4 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = get(r4 * 4 + j) * inv;
        *reinterpret_cast<bf16x4*>(og + d0[r4]) = __builtin_convertvector(f, bf16x4);
      }
      if (p.lse && lse_lane) p.lse[orow] = lse_nat;
    } else {
      const size_t prow = static_cast<size_t>(split) * p.total_q * H + orow;
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 4 * runs; ++j) amax = fmaxf(amax, fabsf(get(j) * inv));
      amax = row_max(amax);
      int e2 = 0;
      if (amax > 32768.f) {
        int fe;
        frexpf(amax, &fe);  // amax <= 2^fe
        e2 = fe - 15;
      }
      const float down = __builtin_ldexpf(inv, -e2);
      _Float16* po = p.part_o16 + prow * D;
#pragma unroll
      for (int r4 = 0; r4 < runs; ++r4) {
        floatx4 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = get(r4 * 4 + j) * down;
        *reinterpret_cast<halfx4*>(po + d0[r4]) = __builtin_convertvector(f, halfx4);
      }
      if (lse_lane) {
        p.part_lse[prow] = lse_nat;
        p.part_scale[prow] = __builtin_ldexpf(1.f, e2);
      }
    }
  };

  // The lane indices are formed again here (from an opaque copy of the
  // thread index) rather than kept alive across the key loop.
  int t_end = tid;
  asm volatile("" : "+v"(t_end));
  {
    const int lane = t_end & 63;
    const int lr = lane & 31, lh = lane >> 5;
    const int c16 = lane & 15, g4 = lane >> 4;
    const int qrow = wrow0 + lr;
    const bool qvalid = qrow < qn;
    // Combine the two tile-parity states of each block, and the extra block's
    // four quarter states, through LDS over the idle ring: every issued tile has
    // been consumed, and the barrier orders the reuse.
    float* const mbuf = reinterpret_cast<float*>(smem);  // [NB][34][64]
    float* const xbuf = mbuf + NB * 34 * 64;             // [3][18][64]
    floatx4 xo[4] = {};
    if (XB && xactive) {
#pragma unroll
      for (int db = 0; db < 4; ++db) xo[db] = lds_xo[(wave * 4 + db) * 64 + lane];
    }
    // (vmcnt: the query loads are still in flight when a split has no tiles)
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    __builtin_amdgcn_s_barrier();
    if (odd && active) {
      float* b = mbuf + blk * 34 * 64 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        b[r * 64] = o0[r];
        b[(16 + r) * 64] = o1[r];
      }
      b[32 * 64] = m_run;
      b[33 * 64] = l_run;
    }
    if (XB && xactive && wave >= 1) {
      float* b = xbuf + (wave - 1) * 18 * 64 + lane;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) b[(db * 4 + i) * 64] = xo[db][i];
      b[16 * 64] = xm;
      b[17 * 64] = xl;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    __builtin_amdgcn_s_barrier();
    if (!odd && active) {
      const float* b = mbuf + blk * 34 * 64 + lane;
      const float m1 = b[32 * 64], l1 = b[33 * 64];
      const float M = fmaxf(m_run, m1);
      const float c0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float c1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] = __builtin_fmaf(b[r * 64], c1, o0[r] * c0);
        o1[r] = __builtin_fmaf(b[(16 + r) * 64], c1, o1[r] * c0);
      }
      const float l_tot = pair_sum(__builtin_fmaf(l1, c1, l_run * c0));
      if (qvalid) {
        // 32x32 accumulator: element r of o0 is dim (r>>2)*8 + 4*lh + (r&3); o1 adds 32.
        const int d0[8] = {4 * lh, 8 + 4 * lh, 16 + 4 * lh, 24 + 4 * lh, 32 + 4 * lh, 40 + 4 * lh, 48 + 4 * lh, 56 + 4 * lh};
        write_row(qrow, [&](int j) { return j < 16 ? o0[j] : o1[j - 16]; }, d0, std::integral_constant<int, 8>{}, M, l_tot, lh == 0,
                [](float x) { return pair_max(x); });
      }
    }
    if (XB && xactive && wave == 0) {
      float mw[3], lw[3];
      float M = xm;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        mw[w] = xbuf[(w * 18 + 16) * 64 + lane];
        lw[w] = xbuf[(w * 18 + 17) * 64 + lane];
        M = fmaxf(M, mw[w]);
      }
      const float c0 = xm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(xm - M);
      float cw[3];
      float lt = xl * c0;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        cw[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        lt = __builtin_fmaf(lw[w], cw[w], lt);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = xo[db][i] * c0;
#pragma unroll
          for (int w = 0; w < 3; ++w) a = __builtin_fmaf(xbuf[(w * 18 + db * 4 + i) * 64 + lane], cw[w], a);
          xo[db][i] = a;
        }
      const float l_tot = quad_sum(lt);
      const int xrow = xrow0 + c16;
      if (xrow < qn) {
        // 16x16 accumulator: element i of xo[db] is dim 16*db + 4*g4 + i.
        const int d0[4] = {4 * g4, 16 + 4 * g4, 32 + 4 * g4, 48 + 4 * g4};
        write_row(xrow, [&](int j) { return xo[j >> 2][j & 3]; }, d0, std::integral_constant<int, 4>{}, M, l_tot, g4 == 0,
                  [](float x) { return quad_max(x); });
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 256-row tiles: software-pipelined kernel.
//
// On CDNA4 a wave's vector (VALU) work overlaps matrix products when the
// SIMD has both kinds of work to issue at once; in the attn_bf16_kernel layout
// (each wave: all products of a tile, then its softmax, then the next
// products) the waves of a SIMD tend to fall into the same phase, and products
// and softmax then run one after the other.  Here eight waves (two per
// SIMD, up to 256 registers each) each own 32 query rows of the tile over
// every key tile, with their queries in registers, and interleave their own
// instruction streams:
//  * block 1 of iteration j: the 8 products of tile j+1's scores, issued
//    between the exponentials, bf16 conversion and row sums of the second
//    half (keys 32..63) of tile j;
//  * block 2: the 8 P V products of tile j, issued between the exponentials
//    and conversion of the first half (keys 0..31) of tile j+1.
// Numerics are the attn_bf16_kernel's: S^T = K Q^T on 32x32x16 products,
// probabilities against the running maximum accepted when every lane's sum
// is at most kSumBound (else the tile's scores are formed again from LDS,
// O and the sums rescaled to the tile maximum), P rounded to bf16, fp32
// accumulators, the same partial-output format for key splits.  The K/V ring,
// its direct loads, the swizzle, the V pool slot order and the masking of
// keys past a page's length are shared with the attn_bf16_kernel.
template <class Src>
__global__ __launch_bounds__(512) void attn_pipe_kernel(const Src src) {
  constexpr int W = 8;                   // waves, one per 32-row block
  constexpr int ROWS = W * 32;
  constexpr int LPT = DMA_PER_TILE / W;  // direct loads per wave per tile
  constexpr int SMEM = STAGES * 2 * TILE_ELEMS * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  uint16_t* const lds_t = reinterpret_cast<uint16_t*>(smem);
  const AttnParams& p = attn_base(src);

  // ---- which (sequence, head, split, query tile): as attn_bf16_kernel -----
  int g, qt;
  attn_tile_of(p, blockIdx.x, g, qt);
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
  const float sl2 = p.scale_log2;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int wrow0 = row0 + wave * 32;
  const bool active = wrow0 < qn;  // wave-uniform; idle waves still load and synchronise

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k_pool);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v_pool);
  const size_t page_stride = static_cast<size_t>(H) * P * D;
  const size_t head_off = static_cast<size_t>(h) * P * D;

  // ---- queries -> registers: the B operand of S^T = K Q^T, dims 16st+8lh..+7
  // of row wrow0+lr (rows past the sequence repeat its last row; their
  // outputs are never written).
  bf16x8 qf[4];
  {
    const int row = min(wrow0 + lr, qn - 1);
    const bf16x8* gq = reinterpret_cast<const bf16x8*>(qg + (static_cast<size_t>(q0 + row) * H + h) * D + lh * 8);
#pragma unroll
    for (int st = 0; st < 4; ++st) qf[st] = gq[2 * st];
  }

  // ---- this wave's share of each tile's 16 direct loads (as attn_bf16_kernel)
  int dma_goff[LPT], dma_loff[LPT];
  bool dma_v[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = wave * LPT + j;
    const int is_v = inst >> 3, part = inst & 7;
    const int row = part * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    dma_v[j] = is_v != 0;
    dma_goff[j] = is_v ? row * P + chunk * 8 : row * D + chunk * 8;
    dma_loff[j] = is_v * TILE_ELEMS + part * 512;
  }
  auto issue = [&](const Cursor& c, int stage) {
    const size_t base = static_cast<size_t>(c.pid) * page_stride + head_off;
    const int koff = c.kt * KT * D, voff = c.kt * KT;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const uint16_t* gp = (dma_v[j] ? vg + voff : kg + koff) + base + dma_goff[j];
      __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds_t + stage * 2 * TILE_ELEMS + dma_loff[j]), 16, 0, 0);
    }
  };
  // Waits for this wave's loads of all tiles but the last `ahead` issued.
  auto wait_tiles = [&](int ahead) {
    if (ahead >= 3)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * LPT));
    else if (ahead == 2)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LPT));
    else if (ahead == 1)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(LPT));
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  };
  // Zero the V^T slots of keys nk..63 of a staged tile (pool slot order, then
  // the chunk swizzle), as attn_bf16_kernel.
  auto zero_tail = [&](uint16_t* lv, int nk) {
    for (int it = tid; it < D * 16; it += W * 64) {
      const int row = it >> 4, grp = it & 15;
      const int k0 = grp * 4;
      if (k0 + 4 <= nk) continue;
      const int sg = (grp & ~3) | ((grp & 1) << 1) | ((grp >> 1) & 1);
      const int pos = sg * 4;
      uint16_t* rp = lv + row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k0 + e >= nk) rp[e] = 0;
    }
  };
  auto stage_ptr = [&](int t) { return lds_t + (t % STAGES) * 2 * TILE_ELEMS; };

  // Scores of a tile from LDS (no interleave: first tile and the rare path).
  auto scores = [&](const uint16_t* lk, floatx16& s0, floatx16& s1) {
    bf16x8 kf[8];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      kf[st] = lds_frag(lk, lr, 2 * st + lh);
      kf[4 + st] = lds_frag(lk, 32 + lr, 2 * st + lh);
    }
    s0 = floatx16{};
    s1 = floatx16{};
#pragma unroll
    for (int st = 0; st < 4; ++st) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s0, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[4 + st], qf[st], s1, 0, 0, 0);
  };
  // Keys nk..63 of a tile get -inf scores (32x32 layout: element r of s0 is
  // key (r>>2)*8 + 4lh + (r&3), s1 adds 32).
  auto mask = [&](floatx16& s0, floatx16& s1, int nk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = (r >> 2) * 8 + lh * 4 + (r & 3);
      if (key >= nk) s0[r] = -INFINITY;
      if (key + 32 >= nk) s1[r] = -INFINITY;
    }
  };

  float m_run = -INFINITY;  // running maximum of scaled scores (log2 domain), per query
  float l_run = 0.f;        // this lane's partial row sum
  floatx16 o0 = {}, o1 = {};

  // Softmax state of a tile between the two iterations that form it: the
  // probabilities of keys 0..31 (P^T fragments 0 and 1, bf16) with this
  // lane's sum of them, and the raw scores of keys 32..63.
  struct TileState {
    bf16x8 pa0, pa1;
    float sa;
    floatx16 sb;
  };
  auto first_half = [&](const floatx16& s0, TileState& t) {
    const float nm = -m_run;
    floatx16 e;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, nm));
    t.sa = half_sum(e);
    t.pa0 = to_bf16x8(e, 0);
    t.pa1 = to_bf16x8(e, 8);
  };
  // The rare path: the tile's scores formed again, its maximum taken, O and
  // the sum rescaled, and all its probabilities formed against the new maximum.
  auto rescale_tile = [&](const uint16_t* lk, int nk, TileState& t, bf16x8& pb2, bf16x8& pb3) {
    floatx16 s0, s1;
    scores(lk, s0, s1);
    if (nk < KT) mask(s0, s1, nk);
    const float mx = pair_max(tile_max(s0, s1)) * sl2;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }
    first_half(s0, t);
    const float nm = -m_run;
    floatx16 e;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, nm));
    pb2 = to_bf16x8(e, 0);
    pb3 = to_bf16x8(e, 8);
    return t.sa + half_sum(e);
  };
  // Second half of a tile's probabilities (keys 32..63) against m_run; returns
  // this lane's sum over the whole tile.
  auto second_half = [&](const TileState& t, bf16x8& pb2, bf16x8& pb3) {
    const float nm = -m_run;
    floatx16 e;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(t.sb[r], sl2, nm));
    pb2 = to_bf16x8(e, 0);
    pb3 = to_bf16x8(e, 8);
    return t.sa + half_sum(e);
  };

  // ---- prologue: first tiles in flight, tile 0's scores ---------------------
  Cursor lc, cc, cn;  // next tile to issue, tile j, tile j+1
  cursor_first(src, eb, ee, lc);
  cc = lc;
  int ni = 0;
  for (int s = 0; s < STAGES - 1 && lc.e < ee; ++s) {
    issue(lc, ni % STAGES);
    cursor_next(src, ee, lc);
    ++ni;
  }
  TileState A, B;
  int j = 0;
  if (ni > 0) {
    wait_tiles(ni - 1);
    __builtin_amdgcn_s_barrier();
    int nkc = min(KT, cc.len - cc.kt * KT);
    if (nkc < KT) zero_tail(stage_ptr(0) + TILE_ELEMS, nkc);
    if (active) {
      floatx16 s0, s1;
      scores(stage_ptr(0), s0, s1);
      if (nkc < KT) mask(s0, s1, nkc);
      m_run = pair_max(tile_max(s0, s1)) * sl2;  // exact maximum of the first tile
      first_half(s0, A);
      A.sb = s1;
    }
    cn = cc;
    cursor_next(src, ee, cn);

    // One iteration: finish tile j (state `cur`) and its P V products, form
    // tile j+1's scores into `nxt`.
    auto body = [&](TileState& cur, TileState& nxt) {
      wait_tiles(ni - (j + 2));
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
      __builtin_amdgcn_s_barrier();
      const int nkn = min(KT, cn.len - cn.kt * KT);
      uint16_t* const lkn = stage_ptr(j + 1);
      if (nkn < KT) zero_tail(lkn + TILE_ELEMS, nkn);  // published by the next barrier
      if (active) {
        const uint16_t* lvc = stage_ptr(j) + TILE_ELEMS;
        const float nm = -m_run;
        auto ex = [&](float s) { return __builtin_amdgcn_exp2f(__builtin_fmaf(s, sl2, nm)); };
        // Each block is eight fenced groups: one product, then the exponentials
        // of one score pair, the bf16 conversion and sum of the previous pair,
        // and a share of the fragment reads the next block needs.
        // block 1: tile j+1's scores under tile j's keys 32..63
        bf16x8 kf[8], vf[8];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          kf[st] = lds_frag(lkn, lr, 2 * st + lh);
          kf[4 + st] = lds_frag(lkn, 32 + lr, 2 * st + lh);
        }
        float e0 = ex(cur.sb[0]), e1 = ex(cur.sb[1]);
        __builtin_amdgcn_sched_barrier(0);
        floatx16 n0 = {}, n1 = {};
        bf16x2 c[8];
        float u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i < 4)
            n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i], n0, 0, 0, 0);
          else
            n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i - 4], n1, 0, 0, 0);
          c[i] = cvt2(e0, e1);
          u[i] = e0 + e1;
          if (i < 7) {
            e0 = ex(cur.sb[2 * i + 2]);
            e1 = ex(cur.sb[2 * i + 3]);
          }
          if (i >= 2 && i < 6) {
            const int t = i - 2;
            vf[t] = lds_frag(lvc, lr, 2 * t + lh);
            vf[4 + t] = lds_frag(lvc, 32 + lr, 2 * t + lh);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pb2 = cat4(c[0], c[1], c[2], c[3]);
        bf16x8 pb3 = cat4(c[4], c[5], c[6], c[7]);
        float lt = cur.sa + (((u[0] + u[1]) + (u[2] + u[3])) + ((u[4] + u[5]) + (u[6] + u[7])));
        if (__any(!(lt <= kSumBound))) {
          // Rare: K of tile j is still staged (its stage is refilled one
          // iteration later).
          lt = rescale_tile(stage_ptr(j), min(KT, cc.len - cc.kt * KT), cur, pb2, pb3);
        }
        l_run += lt;
        if (nkn < KT) mask(n0, n1, nkn);
        // block 2: tile j's P V products under tile j+1's keys 0..31
        const float nm2 = -m_run;
        auto ex2 = [&](float s) { return __builtin_amdgcn_exp2f(__builtin_fmaf(s, sl2, nm2)); };
        __builtin_amdgcn_sched_barrier(0);
        float f0 = ex2(n0[0]), f1 = ex2(n0[1]);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 pb[4] = {cur.pa0, cur.pa1, pb2, pb3};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (t < 4)
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pb[t], o0, 0, 0, 0);
          else
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pb[t - 4], o1, 0, 0, 0);
          c[t] = cvt2(f0, f1);
          u[t] = f0 + f1;
          if (t < 7) {
            f0 = ex2(n0[2 * t + 2]);
            f1 = ex2(n0[2 * t + 3]);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        nxt.pa0 = cat4(c[0], c[1], c[2], c[3]);
        nxt.pa1 = cat4(c[4], c[5], c[6], c[7]);
        nxt.sa = ((u[0] + u[1]) + (u[2] + u[3])) + ((u[4] + u[5]) + (u[6] + u[7]));
        nxt.sb = n1;
      }
      // Stage (j-1) % STAGES is free (every wave is past iteration j-1).
      if (lc.e < ee) {
        issue(lc, ni % STAGES);
        cursor_next(src, ee, lc);
        ++ni;
      }
      cc = cn;
      cursor_next(src, ee, cn);
      ++j;
    };

    // Two iterations per trip so that the two states swap roles without copies.
    while (cn.e < ee) {
      body(A, B);
      if (cn.e >= ee) {
        A = B;
        break;
      }
      body(B, A);
    }

    // ---- last tile: finish its probabilities and its P V products ---------
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    __builtin_amdgcn_s_barrier();  // publishes the last tile's zeroed V slots
    if (active) {
      bf16x8 pb2, pb3;
      float lt = second_half(A, pb2, pb3);
      if (__any(!(lt <= kSumBound))) lt = rescale_tile(stage_ptr(j), min(KT, cc.len - cc.kt * KT), A, pb2, pb3);
      l_run += lt;
      const uint16_t* lvc = stage_ptr(j) + TILE_ELEMS;
      const bf16x8 pb[4] = {A.pa0, A.pa1, pb2, pb3};
#pragma unroll
      for (int t = 0; t < 4; ++t) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag(lvc, lr, 2 * t + lh), pb[t], o0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t) o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_frag(lvc, 32 + lr, 2 * t + lh), pb[t], o1, 0, 0, 0);
    }
  }

  // ---- epilogue: each wave owns its rows; same output forms as attn_bf16_kernel
  if (!active) return;
  int t_end = tid;
  asm volatile("" : "+v"(t_end));
  const int lane2 = t_end & 63;
  const int lr2 = lane2 & 31, lh2 = lane2 >> 5;
  const int qrow = wrow0 + lr2;
  const float ltot = pair_sum(l_run);
  if (qrow >= qn) return;
  const bool empty = !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse_nat = empty ? -INFINITY : (m_run + __log2f(ltot)) * 0.69314718055994530942f;
  const size_t orow = static_cast<size_t>(q0 + qrow) * H + h;
  // 32x32 accumulator: element r of o0 is dim (r>>2)*8 + 4*lh + (r&3); o1 adds 32.
  auto get = [&](int jj) { return jj < 16 ? o0[jj] : o1[jj - 16]; };
  if (p.num_splits == 1) {
    uint16_t* og = static_cast<uint16_t*>(p.o) + orow * D;
#pragma unroll
    for (int r4 = 0; r4 < 8; ++r4) {
      floatx4 f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) f[jj] = get(r4 * 4 + jj) * inv;
      *reinterpret_cast<bf16x4*>(og + r4 * 8 + 4 * lh2) = __builtin_convertvector(f, bf16x4);
    }
    if (p.lse && lh2 == 0) p.lse[orow] = lse_nat;
  } else {
    // Partial O in fp16 as O * 2^-E, E >= 0 the smallest exponent keeping the
    // row's largest magnitude within 2^15, 2^E beside the lse.
    const size_t prow = static_cast<size_t>(split) * p.total_q * H + orow;
    float amax = 0.f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) amax = fmaxf(amax, fabsf(get(jj) * inv));
    amax = pair_max(amax);
    int e2 = 0;
    if (amax > 32768.f) {
      int fe;
      frexpf(amax, &fe);
      e2 = fe - 15;
    }
    const float down = __builtin_ldexpf(inv, -e2);
    _Float16* po = p.part_o16 + prow * D;
#pragma unroll
    for (int r4 = 0; r4 < 8; ++r4) {
      floatx4 f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) f[jj] = get(r4 * 4 + jj) * down;
      *reinterpret_cast<halfx4*>(po + r4 * 8 + 4 * lh2) = __builtin_convertvector(f, halfx4);
    }
    if (lh2 == 0) {
      p.part_lse[prow] = lse_nat;
      p.part_scale[prow] = __builtin_ldexpf(1.f, e2);
    }
  }
}

// ---------------------------------------------------------------------------
// 512-row tiles: eight waves, each owning 64 query rows (two 32-row blocks A
// and B) over every key tile.
//
// The 8-wave kernel above is bound by instruction issue, not by the matrix
// core: per 32x64 unit a wave issues its softmax (about 130 VALU
// instructions) but also the tile's fragment reads, the table walk and
// ring bookkeeping (about 69 SALU and 16 LDS instructions), a direct load and
// a barrier.  Here one wave serves two 32-row blocks with the same K and V
// fragments, the same table walk and the same barrier, so that work is spent
// once per 64 rows.  There is no cross-tile pipeline (the two blocks'
// accumulators take the registers).  Within a tile the score products of
// both blocks are issued together, then block A's softmax and P V products,
// then block B's, so that block A's products can run under block B's
// softmax.  Numerics, ring, masking and output formats are those of the
// other bf16 kernels.  With FP8 pages (KV8) the ring stages codes and row
// exponents; at iteration j the workgroup converts tile j+1 into one of two
// bf16 tiles (as attn_bf16_kernel does for its pairs) before the products on
// tile j, and the next barrier publishes it.
template <class Src, bool KV8 = false>
__global__ __launch_bounds__(512) void attn_wide_kernel(const Src src) {
  constexpr int W = 8;                   // waves, one per 64-row pair of blocks
  constexpr int ROWS = W * 64;
  constexpr int LPT = DMA_PER_TILE / W;  // direct loads per wave per tile
  constexpr int TILE_BYTES = 2 * TILE_ELEMS * 2;   // K and V^T of one bf16 tile
  constexpr int STAGE8 = 2 * TILE_ELEMS + 2 * KT;  // FP8 stage: K codes, V codes, K exps, V exps
  // bf16 pages: the ring of bf16 tiles.  FP8 pages: two converted bf16 tiles
  // (tile j in buffer j % 2), then the ring of FP8 stages.
  constexpr int SMEM = KV8 ? 2 * TILE_BYTES + STAGES * STAGE8 : STAGES * TILE_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  uint16_t* const lds_t = reinterpret_cast<uint16_t*>(smem);
  uint8_t* const lds8 = smem + (KV8 ? 2 * TILE_BYTES : 0);
  const AttnParams& p = attn_base(src);

  // ---- which (sequence, head, split, query tile): as attn_bf16_kernel -----
  int g, qt;
  attn_tile_of(p, blockIdx.x, g, qt);
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
  const float sl2 = p.scale_log2;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int wrow0 = row0 + wave * 64;  // block A: wrow0..+31, block B: wrow0+32..+63
  const bool active = wrow0 < qn;      // wave-uniform; idle waves still load and synchronise

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k_pool);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v_pool);
  const size_t page_stride = static_cast<size_t>(H) * P * D;
  const size_t head_off = static_cast<size_t>(h) * P * D;

  // ---- queries -> registers (B operands of S^T = K Q^T, dims 16st+8lh..+7);
  // rows past the sequence repeat its last row, their outputs are never written.
  bf16x8 qa[4], qb[4];
  {
    const int ra = min(wrow0 + lr, qn - 1), rb = min(wrow0 + 32 + lr, qn - 1);
    const bf16x8* ga = reinterpret_cast<const bf16x8*>(qg + (static_cast<size_t>(q0 + ra) * H + h) * D + lh * 8);
    const bf16x8* gb = reinterpret_cast<const bf16x8*>(qg + (static_cast<size_t>(q0 + rb) * H + h) * D + lh * 8);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      qa[st] = ga[2 * st];
      qb[st] = gb[2 * st];
    }
  }

  // ---- this wave's share of each tile's 16 direct loads (as attn_bf16_kernel)
  int dma_goff[LPT], dma_loff[LPT];
  bool dma_v[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = wave * LPT + j;
    const int is_v = inst >> 3, part = inst & 7;
    const int row = part * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    dma_v[j] = is_v != 0;
    dma_goff[j] = is_v ? row * P + chunk * 8 : row * D + chunk * 8;
    dma_loff[j] = is_v * TILE_ELEMS + part * 512;
  }
  // FP8 loads (as attn_bf16_kernel): inst 0-3 K codes (1 KiB each), 4-7 V
  // codes, 8-11 K exponents and 12-15 V exponents (16 bytes, lane 0 only).
  int dma8_kind[LPT], dma8_off[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int inst = wave * LPT + j;
    const int kind = inst >> 2, q = inst & 3;
    dma8_kind[j] = kind;
    dma8_off[j] = kind < 2 ? kind * 4096 + q * 1024 : 8192 + (kind - 2) * KT + q * 16;
  }
  const uint8_t* __restrict__ kg8 = static_cast<const uint8_t*>(p.k_pool);
  const uint8_t* __restrict__ vg8 = static_cast<const uint8_t*>(p.v_pool);
  const size_t codes_bytes = static_cast<size_t>(p.num_pool_pages) * H * P * D;  // exponents follow
  auto issue = [&](const Cursor& c, int stage) {
    if constexpr (KV8) {
      const size_t row0 = (static_cast<size_t>(c.pid) * H + h) * P + c.kt * KT;  // first slot row of the tile
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int kind = dma8_kind[j];
        const uint8_t* base = (kind & 1) ? vg8 : kg8;
        if (kind < 2) {
          const void* gp = base + row0 * D + (dma8_off[j] & 4095) + lane * 16;
          __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds8 + stage * STAGE8 + dma8_off[j]), 16, 0, 0);
        } else if (lane == 0) {
          const void* gp = base + codes_bytes + row0 + (dma8_off[j] - 8192 - (kind - 2) * KT);
          __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds8 + stage * STAGE8 + dma8_off[j]), 16, 0, 0);
        }
      }
    } else {
      const size_t base = static_cast<size_t>(c.pid) * page_stride + head_off;
      const int koff = c.kt * KT * D, voff = c.kt * KT;
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const uint16_t* gp = (dma_v[j] ? vg + voff : kg + koff) + base + dma_goff[j];
        __builtin_amdgcn_global_load_lds(gp, (lds_void*)(lds_t + stage * 2 * TILE_ELEMS + dma_loff[j]), 16, 0, 0);
      }
    }
  };
  // FP8: converts staged tile `stage` (nk valid keys) into bf16 buffer `b`.
  // Each thread takes one K item, a (token, 8-dim chunk) converted into one
  // 16-byte row write, and one V item, 4 consecutive tokens x 2 dims: the
  // pool slot order keeps each aligned run of 4 slots contiguous, so each of
  // the 2 dims is one 8-byte write of 4 slots into its V^T row (with the chunk
  // swizzle).  Every thread does the same work.  Keys past nk become zeros.
  auto convert = [&](int stage, int b, int nk) {
    const uint8_t* st8 = lds8 + stage * STAGE8;
    uint16_t* tk = lds_t + b * 2 * TILE_ELEMS;
    int t0 = tid;
    asm volatile("" : "+v"(t0));
    // 8 codes of token r, dims 8ch..8ch+7, as 4 words of two bf16 each
    auto dequant = [&](int off, int r, int ch, uint32_t (&u)[4]) {
      const uint2 w = *reinterpret_cast<const uint2*>(st8 + off + r * D + ch * 8);
      const int e = static_cast<int8_t>(st8[8192 + (off ? KT : 0) + r]);
      const float sc = __builtin_ldexpf(1.f, e);
      bf16x2 v2[4];
      v2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.x), sc, false);
      v2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.x), sc, true);
      v2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.y), sc, false);
      v2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w.y), sc, true);
      __builtin_memcpy(u, v2, sizeof u);
      if (r >= nk) u[0] = u[1] = u[2] = u[3] = 0u;
    };
    for (int it = t0; it < KT * 8; it += W * 64) {
      {
        const int r = it >> 3, ch = it & 7;
        uint32_t u[4];
        dequant(0, r, ch, u);
        *reinterpret_cast<uint4*>(tk + r * D + ((ch ^ swz(r)) << 3)) = make_uint4(u[0], u[1], u[2], u[3]);
      }
      {
        // V: tokens r0..r0+3, dims d0, d0+1 (a quarter of an 8-dim chunk)
        const int r0 = (it >> 5) * 4, d0 = (it & 31) * 2;
        uint32_t v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = r0 + t;
          const int w = *reinterpret_cast<const uint16_t*>(st8 + 4096 + r * D + d0);
          const int e = static_cast<int8_t>(st8[8192 + KT + r]);
          const bf16x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, __builtin_ldexpf(1.f, e), false);
          __builtin_memcpy(&v[t], &c2, 4);
          if (r >= nk) v[t] = 0u;
        }
        const int pos = v_slot_pos(r0);  // slots r0..r0+3 sit at pos..pos+3
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = d0 + i;  // dim
          const int sh = 16 * i;
          const uint32_t lo = ((v[0] >> sh) & 0xFFFFu) | (((v[1] >> sh) & 0xFFFFu) << 16);
          const uint32_t hi = ((v[2] >> sh) & 0xFFFFu) | (((v[3] >> sh) & 0xFFFFu) << 16);
          *reinterpret_cast<uint2*>(tk + TILE_ELEMS + row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7))) =
              make_uint2(lo, hi);
        }
      }
    }
  };
  // Waits for this wave's loads of all tiles but the last `ahead` issued.
  auto wait_tiles = [&](int ahead) {
    if (ahead >= 4)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 * LPT));
    else if (ahead == 3)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * LPT));
    else if (ahead == 2)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LPT));
    else if (ahead == 1)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(LPT));
    else
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  };
  // Zero the V^T slots of keys nk..63 of a staged tile (as attn_bf16_kernel).
  auto zero_tail = [&](uint16_t* lv, int nk) {
    for (int it = tid; it < D * 16; it += W * 64) {
      const int row = it >> 4, grp = it & 15;
      const int k0 = grp * 4;
      if (k0 + 4 <= nk) continue;
      const int sg = (grp & ~3) | ((grp & 1) << 1) | ((grp >> 1) & 1);
      const int pos = sg * 4;
      uint16_t* rp = lv + row * D + ((((pos >> 3) ^ swz(row)) << 3) | (pos & 7));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k0 + e >= nk) rp[e] = 0;
    }
  };
  auto stage_ptr = [&](int t) { return lds_t + (KV8 ? (t & 1) : t % STAGES) * 2 * TILE_ELEMS; };
  // Keys nk..63 get -inf scores (32x32 layout: element r of s0 is key
  // (r>>2)*8 + 4lh + (r&3), s1 adds 32); the lane threshold is formed at each
  // call so that no per-element key indices stay live across the loop.
  auto mask = [&](floatx16& s0, floatx16& s1, int nk) {
    int th = nk - 4 * ((tid >> 5) & 1);
    asm volatile("" : "+v"(th));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kb = (r >> 2) * 8 + (r & 3);
      if (kb >= th) s0[r] = -INFINITY;
      if (kb + 32 >= th) s1[r] = -INFINITY;
    }
  };
  // Scores of one block (queries qv) against the tile's K fragments.
  auto scores = [&](const bf16x8 (&kf)[8], const bf16x8 (&qv)[4], floatx16& s0, floatx16& s1) {
    s0 = floatx16{};
    s1 = floatx16{};
#pragma unroll
    for (int st = 0; st < 4; ++st) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qv[st], s0, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[4 + st], qv[st], s1, 0, 0, 0);
  };
  auto kfrags = [&](const uint16_t* lk, bf16x8 (&kf)[8]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      kf[st] = lds_frag(lk, lr, 2 * st + lh);
      kf[4 + st] = lds_frag(lk, 32 + lr, 2 * st + lh);
    }
  };

  // Per block: running maximum (log2 domain, per query), this lane's partial
  // row sum, O^T accumulators (dims 0..31 and 32..63).
  float ma = -INFINITY, mb = -INFINITY, la = 0.f, lb = 0.f;
  floatx16 oa0 = {}, oa1 = {}, ob0 = {}, ob1 = {};

  // Probabilities of one block against its running maximum m, in place, as
  // bf16 P^T fragments; returns this lane's sum.  On the block's first tile m
  // starts at the tile's exact maximum; when a lane's sum exceeds kSumBound
  // the tile's scores are formed again from LDS, m moves to the tile maximum
  // and O and the sum are rescaled (as attn_bf16_kernel).
  auto softmax = [&](floatx16& s0, floatx16& s1, float& m, float& l, floatx16& o0, floatx16& o1,
                     const uint16_t* lk, const bf16x8 (&qv)[4], int nk, bool first, bf16x8 (&pb)[4]) {
    if (first) m = pair_max(tile_max(s0, s1)) * sl2;  // every tile holds at least one valid key
    auto probs = [&]() {
      const float nm = -m;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, nm));
        s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, nm));
      }
      return tile_sum(s0, s1);
    };
    float lt = probs();
    if (__any(!(lt <= kSumBound))) {
      bf16x8 kf[8];
      kfrags(lk, kf);
      scores(kf, qv, s0, s1);
      if (nk < KT) mask(s0, s1, nk);
      const float m_new = fmaxf(m, pair_max(tile_max(s0, s1)) * sl2);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] *= alpha;
        o1[r] *= alpha;
      }
      lt = probs();
    }
    l += lt;
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[t] = to_bf16x8(t < 2 ? s0 : s1, 8 * (t & 1));
  };
  // Probabilities of elements b..b+3 of s against -nm's maximum, in place;
  // returns their sum.
  auto probs4 = [&](floatx16& s, int b, float nm) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[b + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b + r], sl2, nm));
    return (s[b] + s[b + 1]) + (s[b + 2] + s[b + 3]);
  };
  // Rare path of the interleaved tile: as softmax() when the lane sum is out of bounds.
  auto rescale = [&](floatx16& s0, floatx16& s1, float& m, float& l, floatx16& o0, floatx16& o1,
                     const uint16_t* lk, const bf16x8 (&qv)[4], int nk) {
    bf16x8 kf[8];
    kfrags(lk, kf);
    scores(kf, qv, s0, s1);
    if (nk < KT) mask(s0, s1, nk);
    const float m_new = fmaxf(m, pair_max(tile_max(s0, s1)) * sl2);
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }
    const float nm = -m;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sl2, nm));
      s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sl2, nm));
    }
    return tile_sum(s0, s1);
  };
  // One tile with each block's softmax issued beside the other block's
  // products, so that every wave keeps both the matrix core and the VALU fed
  // whatever phase the other wave of its SIMD is in: the tile is laid out as
  // fenced groups of one product plus a four-element slice of a softmax:
  //   block A's 8 score products; 8 x (one of block B's score products, a
  //   slice of block A's softmax); rare path A; block A's probabilities to
  //   bf16 and the V fragments; 8 x (one of block A's P V products, a slice
  //   of block B's softmax); rare path B; block B's 8 P V products.
  auto tile_interleaved = [&](const uint16_t* lk, int nk, bool first) {
    bf16x8 kf[8];
    kfrags(lk, kf);
    floatx16 sa0 = {}, sa1 = {}, sb0 = {}, sb1 = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) sa0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qa[st], sa0, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) sa1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[4 + st], qa[st], sa1, 0, 0, 0);
    if (nk < KT) mask(sa0, sa1, nk);
    if (first) ma = pair_max(tile_max(sa0, sa1)) * sl2;  // every tile holds a valid key
    __builtin_amdgcn_sched_barrier(0);
    float ps[8];
    const float nma = -ma;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < 4)
        sb0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qb[i], sb0, 0, 0, 0);
      else
        sb1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qb[i - 4], sb1, 0, 0, 0);
      ps[i] = probs4(i < 4 ? sa0 : sa1, 4 * (i & 3), nma);
      __builtin_amdgcn_sched_barrier(0);
    }
    float lta = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    if (__any(!(lta <= kSumBound))) lta = rescale(sa0, sa1, ma, la, oa0, oa1, lk, qa, nk);
    la += lta;
    if (nk < KT) mask(sb0, sb1, nk);
    if (first) mb = pair_max(tile_max(sb0, sb1)) * sl2;
    bf16x8 pa[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) pa[t] = to_bf16x8(t < 2 ? sa0 : sa1, 8 * (t & 1));
    const uint16_t* lv = lk + TILE_ELEMS;
    bf16x8 vf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      vf[t] = lds_frag(lv, lr, 2 * t + lh);
      vf[4 + t] = lds_frag(lv, 32 + lr, 2 * t + lh);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float nmb = -mb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < 4)
        oa0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pa[i], oa0, 0, 0, 0);
      else
        oa1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pa[i - 4], oa1, 0, 0, 0);
      ps[i] = probs4(i < 4 ? sb0 : sb1, 4 * (i & 3), nmb);
      __builtin_amdgcn_sched_barrier(0);
    }
    float ltb = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    if (__any(!(ltb <= kSumBound))) ltb = rescale(sb0, sb1, mb, lb, ob0, ob1, lk, qb, nk);
    lb += ltb;
    bf16x8 pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) pb[t] = to_bf16x8(t < 2 ? sb0 : sb1, 8 * (t & 1));
#pragma unroll
    for (int t = 0; t < 4; ++t) ob0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], pb[t], ob0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) ob1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 + t], pb[t], ob1, 0, 0, 0);
  };

  // ---- the key loop: tile j lives in stage j % STAGES ------------------------
  Cursor lc, cc;
  cursor_first(src, eb, ee, lc);
  cc = lc;
  int ni = 0, j = 0;
  for (int s = 0; s < STAGES - 1 && lc.e < ee; ++s) {
    issue(lc, ni % STAGES);
    cursor_next(src, ee, lc);
    ++ni;
  }
  if constexpr (KV8) {
    // FP8: tile 0 is converted here; at iteration j the workgroup converts
    // tile j+1 into the other buffer before its products on tile j, so one
    // barrier per tile publishes both the next bf16 tile and the free stage.
    if (ni > 0) {
      wait_tiles(ni - 1);
      __builtin_amdgcn_s_barrier();
      convert(0, 0, min(KT, cc.len - cc.kt * KT));
    }
  }
  while (cc.e < ee) {
    Cursor cn = cc;  // tile j+1 (FP8: converted in this iteration)
    if constexpr (KV8) {
      cursor_next(src, ee, cn);
      wait_tiles(ni - (j + 2));  // tile j+1
    } else {
      wait_tiles(ni - (j + 1));  // tile j
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
    __builtin_amdgcn_s_barrier();
    // Stage (j-1) % STAGES is free (every wave is past iteration j-1; FP8:
    // that stage was converted at iteration j-2).
    if (lc.e < ee) {
      issue(lc, ni % STAGES);
      cursor_next(src, ee, lc);
      ++ni;
    }
    const int nk = min(KT, cc.len - cc.kt * KT);
    uint16_t* const lk = stage_ptr(j);
    if constexpr (KV8) {
      // Buffer (j+1) % 2 was last read at iteration j-1 (barrier above).
      if (cn.e < ee) convert((j + 1) % STAGES, (j + 1) & 1, min(KT, cn.len - cn.kt * KT));
    } else if (nk < KT) {  // rare: a page's last, partial tile
      zero_tail(lk + TILE_ELEMS, nk);
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
      __builtin_amdgcn_s_barrier();
    }
    if (active) tile_interleaved(lk, nk, j == 0);
    cursor_next(src, ee, cc);
    ++j;
  }

  // ---- epilogue: each wave owns its rows; same output forms as attn_bf16_kernel
  if (!active) return;
  int t_end = tid;
  asm volatile("" : "+v"(t_end));
  const int lr2 = t_end & 31, lh2 = (t_end >> 5) & 1;
  auto write_block = [&](int qrow, const floatx16& o0, const floatx16& o1, float m, float l) {
    const float ltot = pair_sum(l);
    if (qrow >= qn) return;  // (both lanes of a row pair share qrow)
    const bool empty = !(ltot > 0.f);
    const float inv = empty ? 0.f : 1.f / ltot;
    const float lse_nat = empty ? -INFINITY : (m + __log2f(ltot)) * 0.69314718055994530942f;
    const size_t orow = static_cast<size_t>(q0 + qrow) * H + h;
    // 32x32 accumulator: element r of o0 is dim (r>>2)*8 + 4*lh + (r&3); o1 adds 32.
    auto get = [&](int jj) { return jj < 16 ? o0[jj] : o1[jj - 16]; };
    if (p.num_splits == 1) {
      uint16_t* og = static_cast<uint16_t*>(p.o) + orow * D;
#pragma unroll
      for (int r4 = 0; r4 < 8; ++r4) {
        floatx4 f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) f[jj] = get(r4 * 4 + jj) * inv;
        *reinterpret_cast<bf16x4*>(og + r4 * 8 + 4 * lh2) = __builtin_convertvector(f, bf16x4);
      }
      if (p.lse && lh2 == 0) p.lse[orow] = lse_nat;
    } else {
      const size_t prow = static_cast<size_t>(split) * p.total_q * H + orow;
      float amax = 0.f;
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) amax = fmaxf(amax, fabsf(get(jj) * inv));
      amax = pair_max(amax);
      int e2 = 0;
      if (amax > 32768.f) {
        int fe;
        frexpf(amax, &fe);
        e2 = fe - 15;
      }
      const float down = __builtin_ldexpf(inv, -e2);
      _Float16* po = p.part_o16 + prow * D;
#pragma unroll
      for (int r4 = 0; r4 < 8; ++r4) {
        floatx4 f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) f[jj] = get(r4 * 4 + jj) * down;
        *reinterpret_cast<halfx4*>(po + r4 * 8 + 4 * lh2) = __builtin_convertvector(f, halfx4);
      }
      if (lh2 == 0) {
        p.part_lse[prow] = lse_nat;
        p.part_scale[prow] = __builtin_ldexpf(1.f, e2);
      }
    }
  };
  write_block(wrow0 + lr2, oa0, oa1, ma, la);
  write_block(wrow0 + 32 + lr2, ob0, ob1, mb, lb);
}

}  // namespace

// blocks <= 8: that many 32-row blocks; 9: eight blocks plus the shared 16-row
// extra block; 10: sixteen blocks, two per wave (attn_wide_kernel).
int attn_bf16_rows_per_tile(int blocks) { return blocks <= 8 ? blocks * 32 : blocks == 9 ? 8 * 32 + 16 : 512; }

template <bool KV8, class Src>
static hipError_t launch_impl(const Src& src, int waves, hipStream_t stream) {
  const AttnParams& p = attn_base(src);
  const dim3 grid(static_cast<unsigned>(p.q_tiles) * p.groups_padded);
  switch (waves) {
#define KVC_CASE(W)                                                                                    \
  case W:                                                                                              \
    hipLaunchKernelGGL((attn_bf16_kernel<W, false, Src, KV8>), grid, dim3(W * 128), 0, stream, src); \
    break;
    KVC_CASE(1)
    KVC_CASE(2)
    KVC_CASE(3)
    KVC_CASE(4)
    KVC_CASE(5)
    KVC_CASE(6)
    KVC_CASE(7)
#undef KVC_CASE
    case 8:
      if constexpr (KV8)
        hipLaunchKernelGGL((attn_bf16_kernel<8, false, Src, KV8>), grid, dim3(8 * 128), 0, stream, src);
      else
        hipLaunchKernelGGL((attn_pipe_kernel<Src>), grid, dim3(8 * 64), 0, stream, src);
      break;
    case 9:
      hipLaunchKernelGGL((attn_bf16_kernel<8, true, Src, KV8>), grid, dim3(8 * 128), 0, stream, src);
      break;
    case 10:
      hipLaunchKernelGGL((attn_wide_kernel<Src, KV8>), grid, dim3(8 * 64), 0, stream, src);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream) {
  return launch_impl<false>(p, waves, stream);
}
hipError_t launch_attn_bf16(const AttnParamsInline& p, int waves, hipStream_t stream) {
  return launch_impl<false>(p, waves, stream);
}
hipError_t launch_attn_fp8kv(const AttnParams& p, int waves, hipStream_t stream) {
  return launch_impl<true>(p, waves, stream);
}
hipError_t launch_attn_fp8kv(const AttnParamsInline& p, int waves, hipStream_t stream) {
  return launch_impl<true>(p, waves, stream);
}

}  // namespace kvc
