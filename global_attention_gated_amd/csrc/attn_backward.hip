// Backward of an attention layer for training (gradients of the gated-SWA or global layer output with respect to
// q, k, v, the gate logits and the two RMSNorm weights), given the forward's output and log-sum-exp.
//
// The forward (ZGCM-1 summaries: onedev.kr "How it works"; jaehun.me "New Approach" and "How Gated SWA Behaves"),
// per (sequence, query head, query i): q_hat = RoPE(RMSNorm(q) w_q), k_hat = bf16(RoPE(RMSNorm(k) w_k)),
// s_ij = q_hat_i . k_hat_j / sqrt(D) over the visible keys (causal; SWA also i - j < W), p = softmax(s),
// A = p v, out = A (.) sigmoid(g) (SWA) or A (global).  With dout given, the chain rule reads:
//   dA = dout (.) sigmoid(g);  dg = dout (.) A (.) sigmoid(g)(1 - sigmoid(g)) = dout (.) out (.) (1 - sigmoid(g))
//   Delta_i = sum_j p_ij dp_ij = dA_i . A_i = dout_i . out_i     (no division by sigmoid(g) anywhere)
//   dp_ij = dA_i . v_j;  ds_ij = p_ij (dp_ij - Delta_i);  p_ij = exp(s_ij - lse_i)
//   dq_hat_i = sum_j ds_ij k_hat_j / sqrt(D);  dk_hat_j = sum_i ds_ij q_hat_i / sqrt(D);  dv_j = sum_i p_ij dA_i
// summed over the query heads of a GQA group for k and v; then back through RoPE (its transpose) and RMSNorm.
// The bf16 rounding of k_hat passes its gradient through unchanged.
//
// Kernels, in launch order:
//   bwd_prep_kernel  per 64-token block of one head: q_hat (fp16, pre-scaled by log2(e)/sqrt(D), the forward's
//                    score operand) and q_hat^T (bf16); dA and dA^T (bf16), Delta, lse in log2 units, dgate;
//                    for the KV heads k_hat (fp16) and k_hat^T (bf16).  Transposes go through LDS.
//   bwd_kv_kernel    key-centric, in two launches (dV, then dK): a work-group owns a block of 128 keys of one
//                    (sequence, KV head) (causal: two blocks, one from each end of the sequence), one wave per 32
//                    keys, and walks the query tiles that see them for each head of the group; dV^T = dA^T P or
//                    dK_hat^T = Q_hat^T dS accumulates in registers (MFMA 32x32x16, scores in fp16 as the forward,
//                    gradient products in bf16 for their range).
//   bwd_q_kernel     query-centric: a work-group owns 32 positions of the 4 heads of a group (one wave each) and
//                    walks the key tiles they see: dQ_hat^T = K_hat^T dS^T.
//   epilogues        the dK and dQ kernels take their rows back through RoPE (its transpose) and RMSNorm in their
//                    epilogues, write bf16 dk / dq and a per-work-group partial of dw_k / dw_q, which
//                    bwd_dw_reduce_kernel sums in a fixed order.
// The three MFMA kernels copy their tiles from the workspace straight into LDS (buffer loads with LDS as the
// destination, one tile ahead, XOR-swizzled images); the prep writes the transposed tensors in the column order
// those images need.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace zg {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16v8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 32;          // query / key tile of the MFMA kernels
constexpr int kG = 4;           // GQA group (query heads per KV head), the one shape the host accepts
constexpr int kPrepTok = 64;    // tokens per prep work-group
constexpr int kPrepTS = 64;     // LDS row (halves) of the prep transpose tiles [128 dims][64 tokens]
// Element (dim d, token column col) of a prep transpose tile: 16-byte chunk col / 8 of row d sits at chunk position
// (col / 8) ^ (d / 8 % 8).  The writes of one instruction (dims 8c + e of 16 lanes c, one token) then fall in 8
// different chunk positions instead of one bank pair (rows 8 apart are 1 KB apart), and a chunk still reads as one
// 16-byte load.
__device__ __forceinline__ int prep_off(int d, int col) {
  return d * kPrepTS + ((((col >> 3) ^ (d >> 3)) & 7) << 3) + (col & 7);
}
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima (no wait)
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + __expf(-g)); }

__device__ __forceinline__ bf16v8 as_bf16v8(const uint4& w) { return __builtin_bit_cast(bf16v8, w); }
__device__ __forceinline__ half8 as_half8(const uint4& w) { return __builtin_bit_cast(half8, w); }

// 8 fp32 of an MFMA C block (regs j0..j0+7) -> bf16 operand fragment
__device__ __forceinline__ bf16v8 c8_to_bf16(const floatx16& c, int j0) {
  return as_bf16v8(make_uint4(pack_bf16(c[j0], c[j0 + 1]), pack_bf16(c[j0 + 2], c[j0 + 3]), pack_bf16(c[j0 + 4], c[j0 + 5]),
                              pack_bf16(c[j0 + 6], c[j0 + 7])));
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS tile images, filled by buffer loads whose destination is LDS (16 bytes per lane at consecutive addresses;
// the lanes pick their source chunks so the images come out XOR-swizzled, and reads of one chunk by 16 lanes of 16
// consecutive rows hit all 64 banks once):
//   row-major [32 rows][128] (q_hat', dA, k_hat, v): 16-byte chunk c of row r at position c ^ (r % 16)
//   transposed [128 rows][32] (q_hat^T, dA^T, k_hat^T): chunk c (8 columns) of row r at position c ^ ((r / 4) % 4)
// The transposed workspace tensors hold, within each group of 16 tokens, the quads of 4 tokens in the order
// 0, 2, 1, 3 (the prep writes them so): the 8 columns 16t + 4hi + {0..3} and 16t + 8 + 4hi + {0..3}, the order in
// which an MFMA C block holds its rows, are then the stored columns 16t + 8hi .. +7, one chunk.
__device__ __forceinline__ int rm_off(int row, int chunk) { return row * kHeadDim + 8 * (chunk ^ (row & 15)); }
__device__ __forceinline__ int tr_off(int row, int chunk) { return row * kT + 8 * (chunk ^ ((row >> 2) & 3)); }

// Tile reads go through vector types, not the uint4 / float4 structs: a struct copy carries no type-based alias
// information, and without it the compiler makes each LDS read wait for every tile load in flight (the next
// tile's included), which would leave nothing of the prefetch.
__device__ __forceinline__ half8 ld_h8(const uint16_t* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ bf16v8 ld_b8(const uint16_t* p) { return *reinterpret_cast<const bf16v8*>(p); }

// A-operand fragment of a transposed tile for k-step t: row `row`, columns 16t + 4hi + {0..3}, 16t + 8 + 4hi +
// {0..3} (pairs with a B operand built from C registers 8t..8t+7)
__device__ __forceinline__ bf16v8 tr_frag(const uint16_t* tile, int row, int t, int hi) {
  return ld_b8(tile + tr_off(row, 2 * t + hi));
}

// LDS reads at a byte address (the LDS offset of an array plus a per-lane byte offset)
typedef __attribute__((address_space(3))) const unsigned char lds_byte;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ half8 lds_h8(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) half8*>((lds_byte*)(uintptr_t)addr);
}
__device__ __forceinline__ bf16v8 lds_b8(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16v8*>((lds_byte*)(uintptr_t)addr);
}

// A load of 16 bytes per lane from a buffer into LDS at m0 + 16 * lane, written out so that the compiler does not
// track it.  Its wait-count pass cannot always tell these writes (into one stage buffer) from the compute's LDS reads
// (of the other), and then waits for each prefetch right after issuing it.  The kernel that uses it orders these
// loads itself: s_waitcnt vmcnt(0) and a barrier before any read of their data.  The compiler's own vector-memory
// waits stay correct (loads complete in order; an untracked younger load only makes them wait longer).
// desc: buffer descriptor; lds: byte address in LDS; both wave-uniform.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t buf_desc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) & 0xffffu;
  const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
  return (u32x4_t){lo, hi, n, 0x00020000u};
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved, and declared clobbered: nothing here keeps it
__device__ __forceinline__ void dma16(const u32x4_t& desc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(desc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Byte offsets of a lane's 16-byte sources when wave w copies the 1 KB blocks 2w, 2w+1 of an 8 KB tile:
// row-major (block j = rows 4j..4j+3; source rows `stride` bytes apart) and transposed (block j = rows 16j..16j+15).
__device__ __forceinline__ uint32_t rm_src(int wave, int jj, int lane, uint32_t stride) {
  const int row = 4 * (2 * wave + jj) + (lane >> 4);
  return (uint32_t)row * stride + 16u * (uint32_t)((lane & 15) ^ (row & 15));
}
__device__ __forceinline__ uint32_t tr_src(int wave, int jj, int lane, uint32_t stride) {
  const int row = 16 * (2 * wave + jj) + (lane >> 2);
  return (uint32_t)row * stride + 16u * (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
}
__device__ __forceinline__ void dma_tile(const __amdgpu_buffer_rsrc_t& r, uint16_t* tile, int wave, const uint32_t (&off)[2]) {
#pragma unroll
  for (int jj = 0; jj < 2; jj++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + (2 * wave + jj) * 512), 16, (int)off[jj], 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ------------------------------------------------------------------------------------------ prep
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t T1[kHeadDim * kPrepTS];
  __shared__ __attribute__((aligned(16))) uint16_t T2[kHeadDim * kPrepTS];
  const int tid = threadIdx.x;
  const int c = tid & 15, rg = tid >> 4;   // 16 lanes per row, 8 dims each; 16 rows per pass
  const int s0 = blockIdx.x * kPrepTok;
  const bool qmode = (int)blockIdx.y < a.B * a.Hq;
  const int bh = qmode ? (int)blockIdx.y : (int)blockIdx.y - a.B * a.Hq;
  const int H = qmode ? a.Hq : a.Hkv;
  const int b = bh / H, h = bh % H;
  float wf[8];
  unpack8(*reinterpret_cast<const uint4*>((qmode ? a.qw : a.kw) + 8 * c), wf);
  const bool gated = a.gate != nullptr;
  constexpr int kPasses = kPrepTok / 16;

  // every input chunk of the thread's 4 rows first (16 loads in flight per thread in q mode), then the math
  uint4 xin[kPasses], din[kPasses], oin[kPasses], gin[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; pass++) {
    const int s = s0 + pass * 16 + rg;
    const uint4 z = make_uint4(0, 0, 0, 0);
    xin[pass] = din[pass] = oin[pass] = gin[pass] = z;
    if (s < a.S) {
      const int64_t irow = (((int64_t)b * a.S + s) * H + h) * kHeadDim + 8 * c;   // [B][S][H][D] input row
      xin[pass] = load_nt16((qmode ? a.q : a.k) + irow);
      if (qmode) {
        din[pass] = load_nt16(a.dout + irow);
        oin[pass] = load_nt16(a.out + irow);
        if (gated) gin[pass] = load_nt16(a.gate + irow);
      }
    }
  }

#pragma unroll
  for (int pass = 0; pass < kPasses; pass++) {
    const int row = pass * 16 + rg;
    const int s = s0 + row;
    const int64_t wrow = ((int64_t)bh * a.Sp + s) * kHeadDim + 8 * c;   // [b][h][Sp][D] workspace row
    uint4 t1 = make_uint4(0, 0, 0, 0), t2 = make_uint4(0, 0, 0, 0);
    if (s < a.S) {
      const int64_t irow = (((int64_t)b * a.S + s) * H + h) * kHeadDim + 8 * c;   // [B][S][H][D] input row
      float f[8];
      unpack8(xin[pass], f);
      norm_rope8_g16_w(f, wf, c, s, a.eps, a.rot_pairs, a.inv_freq_rev);
      if (qmode) {
        float fs[8];
#pragma unroll
        for (int e = 0; e < 8; e++) fs[e] = f[e] * a.q_scale;
        *reinterpret_cast<uint4*>(a.qh16 + wrow) = make_uint4(pack_f16(fs[0], fs[1]), pack_f16(fs[2], fs[3]),
                                                              pack_f16(fs[4], fs[5]), pack_f16(fs[6], fs[7]));
        t1 = pack8(f);
        float d[8], o[8], g[8];
        unpack8(din[pass], d);
        unpack8(oin[pass], o);
        float delta = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) delta += d[e] * o[e];
        if (gated) {
          unpack8(gin[pass], g);
          float dg[8];
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float sg = sigmoidf_(g[e]);
            dg[e] = d[e] * o[e] * (1.0f - sg);
            d[e] *= sg;
          }
          *reinterpret_cast<uint4*>(a.dgate + irow) = pack8(dg);
        }
        t2 = pack8(d);
        *reinterpret_cast<uint4*>(a.da + wrow) = t2;
        delta += __shfl_xor(delta, 8);
        delta += __shfl_xor(delta, 4);
        delta += __shfl_xor(delta, 2);
        delta += __shfl_xor(delta, 1);
        if (c == 0) {
          a.ndelta[(int64_t)bh * a.Sp + s] = -delta;
          a.nlse2[(int64_t)bh * a.Sp + s] = -(a.lse[(int64_t)bh * a.S + s] * kLog2e);
        }
      } else {
        t1 = pack8(f);                                            // k_hat in its bf16 cache form
        *reinterpret_cast<uint4*>(a.kh16 + wrow) = bf16x8_to_f16x8(t1);
      }
    } else {
      if (qmode) {
        *reinterpret_cast<uint4*>(a.qh16 + wrow) = t1;
        *reinterpret_cast<uint4*>(a.da + wrow) = t2;
        if (c == 0) {
          a.ndelta[(int64_t)bh * a.Sp + s] = 0.f;
          a.nlse2[(int64_t)bh * a.Sp + s] = -INFINITY;
        }
      } else {
        *reinterpret_cast<uint4*>(a.kh16 + wrow) = t1;
      }
    }
    const uint16_t* p1 = reinterpret_cast<const uint16_t*>(&t1);
    const uint16_t* p2 = reinterpret_cast<const uint16_t*>(&t2);
    const int qd = (row >> 2) & 3;   // transposed column: quads of 4 tokens in the order 0, 2, 1, 3 per 16
    const int col = (row & ~15) | (4 * (qd == 1 ? 2 : qd == 2 ? 1 : qd)) | (row & 3);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      T1[prep_off(8 * c + e, col)] = p1[e];
      if (qmode) T2[prep_off(8 * c + e, col)] = p2[e];
    }
  }
  __syncthreads();
  // transposed stores: dim row d = tid / 2, tokens 32 (tid & 1) .. +31 (64 bytes)
  const int d = tid >> 1, half = tid & 1;
  const int64_t trow = ((int64_t)bh * kHeadDim + d) * a.Sp + s0 + 32 * half;
  uint16_t* dst1 = qmode ? a.qt : a.kt;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    *reinterpret_cast<uint4*>(dst1 + trow + 8 * k) =
        *reinterpret_cast<const uint4*>(&T1[prep_off(d, 32 * half + 8 * k)]);
    if (qmode)
      *reinterpret_cast<uint4*>(a.dat + trow + 8 * k) =
          *reinterpret_cast<const uint4*>(&T2[prep_off(d, 32 * half + 8 * k)]);
  }
}

// ------------------------------------------------------------------------------------------ dK, dV
// Epilogue of the dK and dQ kernels: the norm / RoPE backward of one row per lane pair, from the MFMA C layout
// (acc[db][j] holds dim d = 32db + 8(j/4) + 4hi + j%4 of the lane's row; lanes l and l ^ 32 hold the two halves).
// acc is sum_j ds k_hat (or sum_i ds q_hat); dy = acc / sqrt(D) goes back through RoPE (its transpose at
// position pos) and RMSNorm (x re-read, r recomputed):
//   dx = w dy / r - x (sum_d w_d dy_d x_d) / (D r^3),   and this row's share of the weight gradient dy x / r.
// dx is written as bf16 at dxrow (null for a row past the sequence, whose acc is zero).  The weight-gradient shares
// of the wave's 32 rows are summed by a butterfly that halves each lane's list at every exchange, leaving dims
// n = 2 l32 and 2 l32 + 1 of the list in lane l32, and stored in red (this wave's 128 floats).
__device__ __forceinline__ void norm_rope_bwd_rows(const floatx16 (&acc)[4], const uint16_t* xrow, const uint16_t* w,
                                                   uint16_t* dxrow, int pos, const BwdArgs& a, int hi, int l32,
                                                   float* red) {
  constexpr float kInvSqrtD = 0.08838834764831845f;   // 1/sqrt(128)
  float dy[64], xv[64], wv[64];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int jq = 0; jq < 4; jq++) {
      const int d = 32 * db + 8 * jq + 4 * hi, n = 16 * db + 4 * jq;
      const uint2 x4 = xrow ? *reinterpret_cast<const uint2*>(xrow + d) : make_uint2(0, 0);
      const uint2 w4 = *reinterpret_cast<const uint2*>(w + d);
      xv[n] = bf16lo(x4.x); xv[n + 1] = bf16hi(x4.x); xv[n + 2] = bf16lo(x4.y); xv[n + 3] = bf16hi(x4.y);
      wv[n] = bf16lo(w4.x); wv[n + 1] = bf16hi(w4.x); wv[n + 2] = bf16lo(w4.y); wv[n + 3] = bf16hi(w4.y);
#pragma unroll
      for (int e = 0; e < 4; e++) dy[n + e] = acc[db][4 * jq + e] * kInvSqrtD;
    }
  // RoPE transpose: pairs (d, d + 1), d even, rotated back by the angle of position pos
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int jq = 0; jq < 4; jq++)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int d = 32 * db + 8 * jq + 4 * hi + e, n = 16 * db + 4 * jq + e;
        if ((d >> 1) < a.rot_pairs) {
          float c, sn;
          rope_cs(pos, a.inv_freq_rev[d >> 1], c, sn);
          const float d0 = dy[n], d1 = dy[n + 1];
          dy[n] = d0 * c + d1 * sn;
          dy[n + 1] = -d0 * sn + d1 * c;
        }
      }
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int n = 0; n < 64; n++) {
    ss += xv[n] * xv[n];
    dot += wv[n] * dy[n] * xv[n];
  }
  ss = xor32_sum(ss);
  dot = xor32_sum(dot);
  const float r = rsqrtf(ss * (1.0f / kHeadDim) + a.eps);
  const float k3 = dot * r * r * r * (1.0f / kHeadDim);
  if (dxrow) {
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int jq = 0; jq < 4; jq++) {
        const int d = 32 * db + 8 * jq + 4 * hi, n = 16 * db + 4 * jq;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = wv[n + e] * dy[n + e] * r - xv[n + e] * k3;
        *reinterpret_cast<uint2*>(dxrow + d) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
      }
  }
  // weight-gradient shares, summed over the wave's 32 rows (lane bits 4..0, one exchange each)
#pragma unroll
  for (int n = 0; n < 64; n++) dy[n] = dy[n] * xv[n] * r;
#pragma unroll
  for (int step = 0; step < 5; step++) {
    const int o = 16 >> step, half = 32 >> step;
    const bool up = (l32 & o) != 0;
#pragma unroll
    for (int i = 0; i < half; i++) {
      const float send = up ? dy[i] : dy[i + half];
      const float keep = up ? dy[i + half] : dy[i];
      dy[i] = keep + __shfl_xor(send, o);
    }
  }
  const int n0 = 2 * l32, db0 = n0 >> 4, j0 = n0 & 15;
  const int d0 = 32 * db0 + 8 * (j0 >> 2) + 4 * hi + (j0 & 3);
  red[d0] = dy[0];
  red[d0 + 1] = dy[1];
}

// One query tile of the key-centric kernels.  The dV kernel needs q_hat' (scores) and dA^T; the dK kernel
// q_hat' (scores), dA (dP) and q_hat^T.
template <bool DK>
struct KvStage {
  uint16_t qs[kT * kHeadDim];           // q_hat' fp16 [32 queries][128], row-major image
  uint16_t xs[DK ? kT * kHeadDim : 8];  // dK: dA bf16 [32][128], row-major image
  uint16_t xts[kHeadDim * kT];          // dV: dA^T, dK: q_hat^T, bf16 [128][32], transposed image
  float nlse2[kT];   // -lse * log2(e) of the tile's queries
  float ndl[kT];     // -Delta
};

// Key-centric: a work-group owns 128 keys of one (sequence, KV head), one wave per 32 keys, and walks the query
// tiles that see them for each head of the group.  DK = false: dV^T += dA^T P.  DK = true: dK_hat^T +=
// q_hat^T dS with dS = P (dP - Delta), dP = dA V^T.  Every MFMA takes one operand from LDS and the other from
// registers (the wave's key rows, or P / dS from the C registers), so two waves per SIMD fit.
template <bool DK>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_kv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) KvStage<DK> st[2];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS destinations of the tile loads
  const int n_units = a.B * a.Hkv;
  const int unit = blockIdx.x % n_units, slot = blockIdx.x / n_units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const bool swa = a.window > 0;
  // Causal layers: a work-group takes two key blocks, nkb-1-slot (the fewest query tiles) and then slot (the
  // most), so that every work-group has the same work and a (sequence, KV head)'s work-groups all run at once.
  // The first block walks its tiles from the last down, the second from its first up: at any time the
  // work-groups of a KV head in their first block read one tile and those in their second block another, so the
  // work-groups on an XCD share every tile they read through its L2.  Windowed layers: one block each, walked
  // from the last tile down.
  const int nkb = (a.S + 127) / 128;
  // one block: kb, walked upward (UP) or downward; inlined once per direction
  auto run = [&](const int kb, auto up_c) {
    constexpr bool up = decltype(up_c)::value;
    const int jb0 = kb * 128;              // the work-group's keys jb0 .. jb0+127
    const int j0 = jb0 + 32 * wave;        // this wave's keys j0 .. j0+31
    const int key = j0 + l32;              // this lane's key (MFMA column)

    // this lane's key row: k_hat fp16 (score operand) and, for dK, v bf16 (dP operand); K-steps of 16 dims
    uint4 kf[8], vf[DK ? 8 : 1];
    {
      const uint16_t* kr = a.kh16 + ((int64_t)unit * a.Sp + key) * kHeadDim + 8 * hi;
#pragma unroll
      for (int t = 0; t < 8; t++) kf[t] = *reinterpret_cast<const uint4*>(kr + 16 * t);
      if constexpr (DK) {
        const int kc = min(key, a.S - 1);
        const uint16_t* vr = a.v + (((int64_t)b * a.S + kc) * a.Hkv + kvh) * kHeadDim + 8 * hi;
#pragma unroll
        for (int t = 0; t < 8; t++) vf[t] = *reinterpret_cast<const uint4*>(vr + 16 * t);
      }
    }
    // The key rows feed the MFMAs straight from these loads.  Retire them here: otherwise the compiler, unable to
    // prove them complete across the loop's back edge, waits for every load in flight (the next tile's prefetch
    // included; the vector-memory counter retires in order) in front of each MFMA that reads them.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    floatx16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int j = 0; j < 16; j++) acc[db][j] = 0.f;

    // query tiles that see some key of the work-group, per head
    const int jb_last = min(jb0 + 127, a.S - 1);
    const int q_end = swa ? min(a.S, jb_last + a.window) : a.S;   // exclusive
    const int qt0 = jb0 / kT, qt1 = (q_end + kT - 1) / kT;
    const int ntiles = max(qt1 - qt0, 0);
    const int n_it = ntiles * kG;
    const int wq_end = swa ? min(a.S, j0 + 31 + a.window) : a.S;   // this wave's visible queries [j0, wq_end)

    // staging: the tiles go from the workspace straight into LDS (2 x 16 bytes per lane and tile); lse / Delta
    // through a register
    float pf = 0.f;
    // lanes 0..31 fetch lse, 32..63 (dK) Delta.  The pointer is picked by arithmetic: a select of the two arguments
    // becomes a load of the pointer from the argument block at a per-lane offset, and its wait in the loop would also
    // wait for the tile loads.
    const float* pf_src = reinterpret_cast<const float*>(
        reinterpret_cast<uintptr_t>(a.nlse2) +
        (tid >= 32 ? reinterpret_cast<uintptr_t>(a.ndelta) - reinterpret_cast<uintptr_t>(a.nlse2) : (uintptr_t)0));
    const uint32_t rm_o[2] = {rm_src(wave, 0, lane, kHeadDim * 2), rm_src(wave, 1, lane, kHeadDim * 2)};
    const uint32_t tr_o[2] = {tr_src(wave, 0, lane, (uint32_t)a.Sp * 2), tr_src(wave, 1, lane, (uint32_t)a.Sp * 2)};
    // the group's heads inside each tile
    auto tile_q0 = [&](int it) { return (up ? qt0 + it / kG : qt1 - 1 - it / kG) * kT; };
    // issue the loads of tile `it` into buffer buf (the tiles lie wholly inside the workspace: q0 + 32 <= Sp)
    auto load_stage = [&](int it, int buf) {
      const int hq = kvh * kG + it % kG;
      const int q0 = tile_q0(it);
      const int64_t bh = (int64_t)b * a.Hq + hq;
      KvStage<DK>& s = st[buf];
      dma_tile(rsrc(a.qh16 + (bh * a.Sp + q0) * kHeadDim, kT * kHeadDim * 2), s.qs, wave, rm_o);
      dma_tile(rsrc((DK ? a.qt : a.dat) + bh * kHeadDim * a.Sp + q0, (uint32_t)(kHeadDim * a.Sp - q0) * 2), s.xts, wave,
               tr_o);
      if constexpr (DK) dma_tile(rsrc(a.da + (bh * a.Sp + q0) * kHeadDim, kT * kHeadDim * 2), s.xs, wave, rm_o);
      if (tid < (DK ? 64 : 32)) pf = pf_src[bh * a.Sp + q0 + (tid & 31)];
    };
    // the small arrays, once their loads are in; the tile loads before them retire with them (in order)
    auto store_stage = [&](int buf) {
      KvStage<DK>& s = st[buf];
      if (tid < 32) s.nlse2[tid] = pf;
      else if (DK && tid < 64) s.ndl[tid - 32] = pf;
    };

    auto compute = [&](int buf, int it) {
      const int q0 = tile_q0(it);
      if (q0 + kT <= j0 || q0 >= wq_end) return;            // no query of the tile sees this wave's keys
      const KvStage<DK>& s = st[buf];
      // C layout: reg j is query q0 + 8(j/4) + 4hi + j%4, column = this lane's key.  The accumulators start from
      // -lse (scores) and -Delta (dP), stored negated, so the MFMAs return s - lse and dP - Delta.
      floatx16 sacc, dpacc;
#pragma unroll
      for (int jq = 0; jq < 4; jq++) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&s.nlse2[8 * jq + 4 * hi]);
        sacc[4 * jq] = l4.x; sacc[4 * jq + 1] = l4.y; sacc[4 * jq + 2] = l4.z; sacc[4 * jq + 3] = l4.w;
        if constexpr (DK) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&s.ndl[8 * jq + 4 * hi]);
          dpacc[4 * jq] = d4.x; dpacc[4 * jq + 1] = d4.y; dpacc[4 * jq + 2] = d4.z; dpacc[4 * jq + 3] = d4.w;
        }
      }
      // the LDS operands are read two k-steps ahead of the MFMAs that use them (the scheduling barriers keep that
      // order: left alone, the compiler reads each operand right before its MFMA and waits for it there)
      if constexpr (DK) {
        half8 qwin[2];
        bf16v8 xwin[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
          qwin[t] = ld_h8(&s.qs[rm_off(l32, 2 * t + hi)]);
          xwin[t] = ld_b8(&s.xs[rm_off(l32, 2 * t + hi)]);
        }
#pragma unroll
        for (int t = 0; t < 8; t++) {
          const half8 qa = qwin[t & 1];
          const bf16v8 xa = xwin[t & 1];
          if (t + 2 < 8) {
            qwin[t & 1] = ld_h8(&s.qs[rm_off(l32, 2 * (t + 2) + hi)]);
            xwin[t & 1] = ld_b8(&s.xs[rm_off(l32, 2 * (t + 2) + hi)]);
          }
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, as_half8(kf[t]), sacc, 0, 0, 0);
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, as_bf16v8(vf[t]), dpacc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // two independent chains (even and odd k-steps) so consecutive MFMAs do not wait on each other
        floatx16 s2;
#pragma unroll
        for (int j = 0; j < 16; j++) s2[j] = 0.f;
        half8 qwin[4];
#pragma unroll
        for (int t = 0; t < 4; t++) qwin[t] = ld_h8(&s.qs[rm_off(l32, 2 * t + hi)]);
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const half8 qa = qwin[t & 3], qb = qwin[(t + 1) & 3];
          if (t + 4 < 8) {
            qwin[t & 3] = ld_h8(&s.qs[rm_off(l32, 2 * (t + 4) + hi)]);
            qwin[(t + 1) & 3] = ld_h8(&s.qs[rm_off(l32, 2 * (t + 5) + hi)]);
          }
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, as_half8(kf[t]), sacc, 0, 0, 0);
          s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(qb, as_half8(kf[t + 1]), s2, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 16; j++) sacc[j] += s2[j];
      }
      // the first four operands of the dV / dK products, read while the exponentials run
      constexpr int TW = DK ? 2 : 4;
      bf16v8 twin[TW];
#pragma unroll
      for (int f = 0; f < TW; f++) twin[f] = tr_frag(s.xts, 32 * (f & 3) + l32, f >> 2, hi);
      // P (dV) or dS = P (dP - Delta) (dK) replaces S; the mask only where the diagonal, the window edge or the
      // sequence end cuts the tile (wave-uniform test)
      const bool inside = q0 >= j0 + 31 && q0 + 31 < a.S && (!swa || q0 + 31 - j0 < a.window) && j0 + 31 < a.S;
      if (inside) {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const float pj = __builtin_amdgcn_exp2f(sacc[j]);
          sacc[j] = DK ? pj * dpacc[j] : pj;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int qi = q0 + 8 * (j >> 2) + 4 * hi + (j & 3);
          const bool vis = qi < a.S && key <= qi && (!swa || qi - key < a.window);
          const float pj = vis ? __builtin_amdgcn_exp2f(sacc[j]) : 0.f;
          sacc[j] = DK ? pj * dpacc[j] : pj;
        }
      }
      const bf16v8 xb[2] = {c8_to_bf16(sacc, 0), c8_to_bf16(sacc, 8)};
#pragma unroll
      for (int f = 0; f < 8; f++) {   // f = 4t + db
        const bf16v8 ta = twin[f % TW];
        if (f + TW < 8) twin[f % TW] = tr_frag(s.xts, 32 * ((f + TW) & 3) + l32, (f + TW) >> 2, hi);
        acc[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, xb[f >> 2], acc[f & 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (n_it > 0) {
      load_stage(0, 0);
      store_stage(0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the tile loads write LDS without the compiler waiting for them
    __syncthreads();
    // Two steps per pass, so that each step's buffer is a constant (with a computed buffer index the compiler waits
    // for the next tile's loads before the compute's first LDS read).
    auto step = [&](int it, int buf) {
      const bool more = it + 1 < n_it;
      if (more) load_stage(it + 1, buf ^ 1);
      compute(buf, it);
      // Keep the stores of the prefetched small arrays after the compute: they go to the other buffer, so the
      // compiler would otherwise move them (and the wait for their loads) up against the loads, which makes the
      // prefetch synchronous.
      asm volatile("" ::: "memory");
      if (more) store_stage(buf ^ 1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    };
    for (int it = 0; it < n_it; it += 2) {
      step(it, 0);
      if (it + 1 < n_it) step(it + 1, 1);
    }

    // outputs: C layout reg j of block db is dim 32db + 8(j/4) + 4hi + j%4 of this lane's key
    if constexpr (DK) {
      // dk: back through RoPE and the key RMSNorm here; the work-group's 128 keys' share of dw_k into its partial
      // the weight-gradient sums in the tile buffers (free after the loop's last barrier): a second LDS array would
      // give the tile reads alias scopes that make them wait for the tile loads in flight
      float (*red)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(&st[0]);
      const int64_t row = ((int64_t)b * a.S + key) * a.Hkv + kvh;
      const bool valid = key < a.S;
      norm_rope_bwd_rows(acc, valid ? a.k + row * kHeadDim : nullptr, a.kw, valid ? a.dk + row * kHeadDim : nullptr,
                         key, a, hi, l32, red[wave]);
      __syncthreads();
      if (tid < kHeadDim)
        a.dw_part[((int64_t)a.n_qblk + (int64_t)kb * n_units + unit) * kHeadDim + tid] =
            red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    } else if (key < a.S) {
      uint16_t* dvr = a.dv + (((int64_t)b * a.S + key) * a.Hkv + kvh) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int jq = 0; jq < 4; jq++) {
          const int d = 32 * db + 8 * jq + 4 * hi;
          *reinterpret_cast<uint2*>(dvr + d) = make_uint2(pack_bf16(acc[db][4 * jq], acc[db][4 * jq + 1]),
                                                          pack_bf16(acc[db][4 * jq + 2], acc[db][4 * jq + 3]));
        }
    }
  };
  if (swa || 2 * slot + 1 == nkb) {
    run(swa ? slot : nkb - 1 - slot, std::false_type{});
  } else {
    run(nkb - 1 - slot, std::false_type{});
    __syncthreads();   // the second block's first tile loads go to the buffer the weight-gradient sums were read from
    run(slot, std::true_type{});
  }
}

// ------------------------------------------------------------------------------------------ dK and dV together
// Causal (global) layers: one kernel forms S and dP once per (key block, query tile) and accumulates both dV^T +=
// dA^T P and dK_hat^T += q_hat^T dS (four products per tile instead of five in the two kernels above, and one set of
// exponentials).  A work-group of 8 waves owns 256 keys (one wave per 32), so that its two gradient accumulators
// fit two waves per SIMD: the wave's k_hat rows stay in registers (score operand) and the block's 256 v rows sit
// in LDS as a row-major image (dP operand), read like the query tiles.
constexpr int kKvfKeys = 256;   // keys per work-group
struct KvfStage {
  uint16_t qs[kT * kHeadDim];    // q_hat' fp16 [32 queries][128], row-major image
  uint16_t xs[kT * kHeadDim];    // dA bf16 [32][128], row-major image
  uint16_t dat[kHeadDim * kT];   // dA^T bf16 [128][32], transposed image
  uint16_t qts[kHeadDim * kT];   // q_hat^T bf16 [128][32], transposed image
  float nlse2[kT];   // -lse * log2(e) of the tile's queries
  float ndl[kT];     // -Delta
};

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_kvf_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vimg[kKvfKeys * kHeadDim];   // v bf16 [256 keys][128], row-major
  __shared__ __attribute__((aligned(16))) KvfStage st[2];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0..7, wave-uniform: LDS destinations of the loads
  const int n_units = a.B * a.Hkv;
  const int unit = blockIdx.x % n_units, slot = blockIdx.x / n_units;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  // key blocks paired as in bwd_kv_kernel: nkb-1-slot walked down, then slot walked up (equal work per work-group)
  const int nkb = (a.S + kKvfKeys - 1) / kKvfKeys;
  // source offsets of this wave's 1 KB blocks: block w of each staged tile (row-major rows 4w..4w+3 are
  // rm_src(w/2, w%2); transposed rows 16w..16w+15 tr_src(w/2, w%2))
  const uint32_t rm_o = rm_src(wave >> 1, wave & 1, lane, kHeadDim * 2);
  const uint32_t tr_o = tr_src(wave >> 1, wave & 1, lane, (uint32_t)a.Sp * 2);
  auto run = [&](const int kb, auto up_c) {
    constexpr bool up = decltype(up_c)::value;
    const int jb0 = kb * kKvfKeys;          // the work-group's keys jb0 .. jb0+255
    const int j0 = jb0 + 32 * wave;         // this wave's keys j0 .. j0+31
    const int key = j0 + l32;               // this lane's key (MFMA column)

    // the block's v rows -> LDS image (row r: chunk c at position c ^ (r % 16)); rows past the sequence read as zero
    {
      const uint32_t vstride = (uint32_t)a.Hkv * kHeadDim * 2;
      // (wave-uniform; readfirstlane keeps the descriptor in scalar registers, which the min / max would not)
      const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kKvfKeys, a.S - jb0)));
      const uint32_t vbytes = rows > 0 ? (uint32_t)(rows - 1) * vstride + kHeadDim * 2 : 0u;
      const u32x4_t rv = buf_desc(a.v + (((int64_t)b * a.S + min(jb0, a.S - 1)) * a.Hkv + kvh) * kHeadDim, vbytes);
#pragma unroll
      for (int jj = 0; jj < 8; jj++) {
        const int blk = 8 * wave + jj, row = 4 * blk + (lane >> 4);
        const uint32_t off = (uint32_t)row * vstride + 16u * (uint32_t)((lane & 15) ^ (row & 15));
        dma16(rv, lds_addr(vimg + blk * 512), off);
      }
    }
    // this lane's k_hat row (fp16, the score operand), K-steps of 16 dims; rows past the workspace clamp to its last
    // row (their scores are masked)
    uint4 kf[8];
    {
      const uint16_t* kr = a.kh16 + ((int64_t)unit * a.Sp + min(key, a.Sp - 1)) * kHeadDim + 8 * hi;
#pragma unroll
      for (int t = 0; t < 8; t++) kf[t] = *reinterpret_cast<const uint4*>(kr + 16 * t);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // retire the preloads (see bwd_kv_kernel)
    floatx16 accv[4], acck[4];
#pragma unroll
    for (int db = 0; db < 4; db++)
#pragma unroll
      for (int j = 0; j < 16; j++) accv[db][j] = acck[db][j] = 0.f;

    const int qt0 = jb0 / kT, qt1 = (a.S + kT - 1) / kT;
    const int n_it = max(qt1 - qt0, 0) * kG;
    float pf = 0.f;
    const float* pf_src = reinterpret_cast<const float*>(
        reinterpret_cast<uintptr_t>(a.nlse2) +
        (tid >= 32 ? reinterpret_cast<uintptr_t>(a.ndelta) - reinterpret_cast<uintptr_t>(a.nlse2) : (uintptr_t)0));
    auto tile_q0 = [&](int it) { return (up ? qt0 + it / kG : qt1 - 1 - it / kG) * kT; };
    auto load_stage = [&](int it, int buf) {
      const int hq = kvh * kG + it % kG;
      const int q0 = tile_q0(it);
      const int64_t bh = (int64_t)b * a.Hq + hq;
      KvfStage& sg = st[buf];
      dma16(buf_desc(a.qh16 + (bh * a.Sp + q0) * kHeadDim, kT * kHeadDim * 2), lds_addr(sg.qs + wave * 512), rm_o);
      dma16(buf_desc(a.da + (bh * a.Sp + q0) * kHeadDim, kT * kHeadDim * 2), lds_addr(sg.xs + wave * 512), rm_o);
      dma16(buf_desc(a.dat + bh * kHeadDim * a.Sp + q0, (uint32_t)(kHeadDim * a.Sp - q0) * 2), lds_addr(sg.dat + wave * 512),
            tr_o);
      dma16(buf_desc(a.qt + bh * kHeadDim * a.Sp + q0, (uint32_t)(kHeadDim * a.Sp - q0) * 2), lds_addr(sg.qts + wave * 512),
            tr_o);
      if (tid < 64) pf = pf_src[bh * a.Sp + q0 + (tid & 31)];
    };
    auto store_stage = [&](int buf) {
      KvfStage& sg = st[buf];
      if (tid < 32) sg.nlse2[tid] = pf;
      else if (tid < 64) sg.ndl[tid - 32] = pf;
    };
    // Fragment addresses.  Row-major images: chunk 2t + hi of row r sits at byte r * 256 + 16 ((2t + hi) ^ (r % 16)),
    // which is (r * 256 + 16 (hi ^ (r % 16))) ^ 32t; the q / dA tiles read row l32, the v image row 32 wave + l32
    // (the same XOR pattern, 8 KB further per wave).  Transposed images: chunk 2t + hi of row 32db + l32 sits at
    // db * 2048 + ((l32 * 64 + 16 (hi ^ ((l32 / 4) % 4))) ^ 32t).  One XOR per read from three per-lane bases.
    const uint32_t rm_b = (uint32_t)l32 * 256u + 16u * (uint32_t)(hi ^ (l32 & 15));
    const uint32_t tr_b = (uint32_t)l32 * 64u + 16u * (uint32_t)(hi ^ ((l32 >> 2) & 3));
    const uint32_t v_b = rm_b + (uint32_t)wave * 8192u;

    auto compute = [&](int buf, int it) {
      const int q0 = tile_q0(it);
      if (q0 + kT <= j0) return;   // every query of the tile is before this wave's keys
      const KvfStage& sg = st[buf];
      // C layout: reg j is query q0 + 8(j/4) + 4hi + j%4, column = this lane's key; the accumulators start from
      // -lse and -Delta (stored negated), so the MFMAs return s - lse and dP - Delta
      floatx16 sacc, dpacc;
#pragma unroll
      for (int jq = 0; jq < 4; jq++) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sg.nlse2[8 * jq + 4 * hi]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sg.ndl[8 * jq + 4 * hi]);
        sacc[4 * jq] = l4.x; sacc[4 * jq + 1] = l4.y; sacc[4 * jq + 2] = l4.z; sacc[4 * jq + 3] = l4.w;
        dpacc[4 * jq] = d4.x; dpacc[4 * jq + 1] = d4.y; dpacc[4 * jq + 2] = d4.z; dpacc[4 * jq + 3] = d4.w;
      }
      // per-lane bases made opaque here, so the compiler derives each address inside the tile (one XOR) instead of
      // holding every fragment's address in a register across the loop
      uint32_t rb = rm_b, tb = tr_b, vbb = v_b;
      asm volatile("" : "+v"(rb), "+v"(tb), "+v"(vbb));
      const uint32_t qs_a = lds_addr(sg.qs), xs_a = lds_addr(sg.xs), v_a = lds_addr(vimg);
      const uint32_t dat_a = lds_addr(sg.dat), qts_a = lds_addr(sg.qts);
      // LDS operands one k-step ahead of their MFMAs (scheduling barriers keep the order; two ahead would not fit
      // the registers without spill reloads in the loop, whose waits would also wait for the prefetch)
      half8 qwin;
      bf16v8 xwin, vwin;
      qwin = lds_h8(qs_a + rb);
      xwin = lds_b8(xs_a + rb);
      vwin = lds_b8(v_a + vbb);
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const half8 qa = qwin;
        const bf16v8 xa = xwin, vb = vwin;
        if (t + 1 < 8) {
          qwin = lds_h8(qs_a + (rb ^ (32u * (t + 1))));
          xwin = lds_b8(xs_a + (rb ^ (32u * (t + 1))));
          vwin = lds_b8(v_a + (vbb ^ (32u * (t + 1))));
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, as_half8(kf[t]), sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, vb, dpacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the first two operands of the dV product, read while the exponentials run
      // transposed-image operand f (f % 8 = 4t + db): dA^T for f < 8, q_hat^T after
      auto tfrag = [&](int f) {
        return lds_b8((f < 8 ? dat_a : qts_a) + 2048u * (uint32_t)(f & 3) + (tb ^ (32u * (uint32_t)((f >> 2) & 1))));
      };
      bf16v8 twin[2];
#pragma unroll
      for (int f = 0; f < 2; f++) twin[f] = tfrag(f);
      // P = exp2(s - lse), masked only where the diagonal or the sequence end cuts the tile (wave-uniform test)
      const bool inside = q0 >= j0 + 31 && q0 + 31 < a.S && j0 + 31 < a.S;
      if (inside) {
#pragma unroll
        for (int j = 0; j < 16; j++) sacc[j] = __builtin_amdgcn_exp2f(sacc[j]);
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const int qi = q0 + 8 * (j >> 2) + 4 * hi + (j & 3);
          sacc[j] = (qi < a.S && key <= qi) ? __builtin_amdgcn_exp2f(sacc[j]) : 0.f;
        }
      }
      const bf16v8 pb[2] = {c8_to_bf16(sacc, 0), c8_to_bf16(sacc, 8)};
#pragma unroll
      for (int j = 0; j < 16; j++) sacc[j] *= dpacc[j];   // dS = P (dP - Delta)
      const bf16v8 sb[2] = {c8_to_bf16(sacc, 0), c8_to_bf16(sacc, 8)};
      // dV^T += dA^T P (f = 0..7), then dK_hat^T += q_hat^T dS (f = 8..15); f % 8 = 4t + db
#pragma unroll
      for (int f = 0; f < 16; f++) {
        const bf16v8 ta = twin[f & 1];
        const int n = f + 2;
        if (n < 16) twin[f & 1] = tfrag(n);
        if (f < 8) accv[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, pb[f >> 2], accv[f & 3], 0, 0, 0);
        else acck[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, sb[(f >> 2) & 1], acck[f & 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (n_it > 0) {
      load_stage(0, 0);
      store_stage(0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the v image and the first tiles, loaded into LDS without compiler waits
    __syncthreads();
    auto step = [&](int it, int buf) {
      const bool more = it + 1 < n_it;
      if (more) load_stage(it + 1, buf ^ 1);
      compute(buf, it);
      asm volatile("" ::: "memory");   // keep the small arrays' stores after the compute (see bwd_kv_kernel)
      if (more) store_stage(buf ^ 1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    };
    for (int it = 0; it < n_it; it += 2) {
      step(it, 0);
      if (it + 1 < n_it) step(it + 1, 1);
    }

    // outputs: C layout reg j of block db is dim 32db + 8(j/4) + 4hi + j%4 of this lane's key
    if (key < a.S) {
      uint16_t* dvr = a.dv + (((int64_t)b * a.S + key) * a.Hkv + kvh) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; db++)
#pragma unroll
        for (int jq = 0; jq < 4; jq++) {
          const int d = 32 * db + 8 * jq + 4 * hi;
          *reinterpret_cast<uint2*>(dvr + d) = make_uint2(pack_bf16(accv[db][4 * jq], accv[db][4 * jq + 1]),
                                                          pack_bf16(accv[db][4 * jq + 2], accv[db][4 * jq + 3]));
        }
    }
    // dk back through RoPE and the key RMSNorm; the block's share of dw_k into its partial (sums in the tile buffers,
    // free after the loop's last barrier)
    float (*red)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(&st[0]);
    const int64_t row = ((int64_t)b * a.S + key) * a.Hkv + kvh;
    const bool valid = key < a.S;
    norm_rope_bwd_rows(acck, valid ? a.k + row * kHeadDim : nullptr, a.kw, valid ? a.dk + row * kHeadDim : nullptr,
                       key, a, hi, l32, red[wave]);
    __syncthreads();
    if (tid < kHeadDim) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 8; w++) sum += red[w][tid];
      a.dw_part[((int64_t)a.n_qblk + (int64_t)kb * n_units + unit) * kHeadDim + tid] = sum;
    }
  };
  if (2 * slot + 1 == nkb) {
    run(slot, std::false_type{});
  } else {
    run(nkb - 1 - slot, std::false_type{});
    __syncthreads();   // the second block's loads go to the v image and the buffers the weight-gradient sums used
    run(slot, std::true_type{});
  }
}

// ------------------------------------------------------------------------------------------ dQ
struct QStage {
  uint16_t ks[kT * kHeadDim];      // k_hat fp16 [32 keys][128], row-major image
  uint16_t vs[kT * kHeadDim];      // v bf16 [32][128], row-major image
  uint16_t kts[kHeadDim * kT];     // k_hat^T bf16 [128][32], transposed image
};

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_q_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) QStage st[2];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS destinations of the tile loads
  const int n_units = a.B * a.Hkv;
  const int n_qt = (a.S + kT - 1) / kT;
  const int unit = blockIdx.x % n_units, rank = blockIdx.x / n_units;
  const bool swa = a.window > 0;
  const int qt = swa ? rank : n_qt - 1 - rank;            // global: longest rows first
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int hq = kvh * kG + wave;
  const int i0 = qt * kT;
  const int qi = i0 + l32;                                 // this lane's query (MFMA column)
  const int64_t bh = (int64_t)b * a.Hq + hq;

  uint4 qf[8], daf[8];
  {
    const uint16_t* qr = a.qh16 + (bh * a.Sp + qi) * kHeadDim + 8 * hi;
    const uint16_t* dr = a.da + (bh * a.Sp + qi) * kHeadDim + 8 * hi;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      qf[t] = *reinterpret_cast<const uint4*>(qr + 16 * t);
      daf[t] = *reinterpret_cast<const uint4*>(dr + 16 * t);
    }
  }
  const float nlse2 = a.nlse2[bh * a.Sp + qi];
  const float ndl = a.ndelta[bh * a.Sp + qi];
  // retire the preloads (see bwd_kv_kernel)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  floatx16 dq[4];
#pragma unroll
  for (int db = 0; db < 4; db++)
#pragma unroll
    for (int j = 0; j < 16; j++) dq[db][j] = 0.f;

  const int k_end = min(a.S, i0 + kT);
  const int k_beg = swa ? max(0, i0 - a.window + 1) : 0;
  const int kt0 = k_beg / kT, kt1 = (k_end + kT - 1) / kT;
  const int n_it = kt1 - kt0;

  // staging: the tiles go from the workspace (k_hat, k_hat^T) and the input (v) straight into LDS, 2 x 16 bytes
  // per lane and tile.  v rows are Hkv * 128 elements apart; the descriptor ends after the sequence's last row, so
  // the rows of a tile past it read zeros (their keys are masked).
  const uint32_t vstride = (uint32_t)a.Hkv * kHeadDim * 2;
  const uint32_t rm_o[2] = {rm_src(wave, 0, lane, kHeadDim * 2), rm_src(wave, 1, lane, kHeadDim * 2)};
  const uint32_t rv_o[2] = {rm_src(wave, 0, lane, vstride), rm_src(wave, 1, lane, vstride)};
  const uint32_t tr_o[2] = {tr_src(wave, 0, lane, (uint32_t)a.Sp * 2), tr_src(wave, 1, lane, (uint32_t)a.Sp * 2)};
  auto load_stage = [&](int it, int buf) {
    const int k0 = (kt0 + it) * kT;
    QStage& s = st[buf];
    dma_tile(rsrc(a.kh16 + ((int64_t)unit * a.Sp + k0) * kHeadDim, kT * kHeadDim * 2), s.ks, wave, rm_o);
    dma_tile(rsrc(a.v + (((int64_t)b * a.S + k0) * a.Hkv + kvh) * kHeadDim,
                  (uint32_t)(a.S - 1 - k0) * vstride + kHeadDim * 2),
             s.vs, wave, rv_o);
    dma_tile(rsrc(a.kt + (int64_t)unit * kHeadDim * a.Sp + k0, (uint32_t)(kHeadDim * a.Sp - k0) * 2), s.kts, wave,
             tr_o);
  };
  auto compute = [&](int buf, int it) {
    const int k0 = (kt0 + it) * kT;
    const QStage& s = st[buf];
    // C layout: reg j is key k0 + 8(j/4) + 4hi + j%4, column = this lane's query; the accumulators start from
    // -lse and -Delta (this lane's query), so the MFMAs return s - lse and dP - Delta
    floatx16 sacc, dpacc;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      sacc[j] = nlse2;
      dpacc[j] = ndl;
    }
    // the LDS operands are read two k-steps ahead of the MFMAs that use them (the scheduling barriers keep that
    // order: left alone, the compiler reads each operand right before its MFMA and waits for it there)
    half8 kwin[2];
    bf16v8 vwin[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      kwin[t] = ld_h8(&s.ks[rm_off(l32, 2 * t + hi)]);
      vwin[t] = ld_b8(&s.vs[rm_off(l32, 2 * t + hi)]);
    }
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const half8 ka = kwin[t & 1];
      const bf16v8 va = vwin[t & 1];
      if (t + 2 < 8) {
        kwin[t & 1] = ld_h8(&s.ks[rm_off(l32, 2 * (t + 2) + hi)]);
        vwin[t & 1] = ld_b8(&s.vs[rm_off(l32, 2 * (t + 2) + hi)]);
      }
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, as_half8(qf[t]), sacc, 0, 0, 0);
      dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16v8(daf[t]), dpacc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first four k_hat^T operands of the dQ products, read while the exponentials run
    bf16v8 twin[4];
#pragma unroll
    for (int f = 0; f < 4; f++) twin[f] = tr_frag(s.kts, 32 * (f & 3) + l32, f >> 2, hi);
    // the mask only where the diagonal, the window edge or the sequence end cuts the tile (wave-uniform test)
    const bool inside = k0 + 31 <= i0 && i0 + 31 < a.S && (!swa || i0 + 31 - k0 < a.window);
    if (inside) {
#pragma unroll
      for (int j = 0; j < 16; j++) sacc[j] = __builtin_amdgcn_exp2f(sacc[j]) * dpacc[j];
    } else {
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int kj = k0 + 8 * (j >> 2) + 4 * hi + (j & 3);
        const bool vis = qi < a.S && kj <= qi && (!swa || qi - kj < a.window);
        sacc[j] = vis ? __builtin_amdgcn_exp2f(sacc[j]) * dpacc[j] : 0.f;
      }
    }
    const bf16v8 sb[2] = {c8_to_bf16(sacc, 0), c8_to_bf16(sacc, 8)};
#pragma unroll
    for (int f = 0; f < 8; f++) {   // f = 4t + db
      const bf16v8 ta = twin[f & 3];
      if (f + 4 < 8) twin[f & 3] = tr_frag(s.kts, 32 * ((f + 4) & 3) + l32, (f + 4) >> 2, hi);
      dq[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, sb[f >> 2], dq[f & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_it > 0) load_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the tile loads write LDS without the compiler waiting for them
  __syncthreads();
  auto step = [&](int it, int buf) {   // two per pass, constant buffers (as in bwd_kv_kernel)
    if (it + 1 < n_it) load_stage(it + 1, buf ^ 1);
    compute(buf, it);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  for (int it = 0; it < n_it; it += 2) {
    step(it, 0);
    if (it + 1 < n_it) step(it + 1, 1);
  }

  // dq: back through RoPE and the query RMSNorm here; the work-group's 4 x 32 rows' share of dw_q into its partial
  float (*red)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(&st[0]);   // in the tile buffers, as in bwd_kv_kernel
  const int64_t row = ((int64_t)b * a.S + qi) * a.Hq + hq;
  const bool valid = qi < a.S;
  norm_rope_bwd_rows(dq, valid ? a.q + row * kHeadDim : nullptr, a.qw, valid ? a.dq + row * kHeadDim : nullptr, qi, a,
                     hi, l32, red[wave]);
  __syncthreads();
  if (tid < kHeadDim)
    a.dw_part[(int64_t)blockIdx.x * kHeadDim + tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

__global__ void __launch_bounds__(128) bwd_dw_zero_kernel(float* dqw, float* dkw) {
  dqw[threadIdx.x] = 0.f;
  dkw[threadIdx.x] = 0.f;
}

// dw_q = sum of the dQ work-groups' partials, dw_k = sum of the dK work-groups'.  Thread t sums the rows
// i = t/128 (mod 8) of dim t%128, sixteen loads in flight, each into its own accumulator; accumulators and then
// the eight slices are added in a fixed order, so the result is deterministic.
__global__ void __launch_bounds__(1024) bwd_dw_reduce_kernel(BwdArgs a) {
  constexpr int kSlices = 8, kLanes = 16;
  __shared__ float red[kSlices][kHeadDim];
  const int kmode = blockIdx.x, d = threadIdx.x & (kHeadDim - 1), slice = threadIdx.x >> 7;
  const float* part = a.dw_part + (kmode ? (int64_t)a.n_qblk * kHeadDim : 0);
  const int n = kmode ? a.n_kblk : a.n_qblk;
  float acc[kLanes];
#pragma unroll
  for (int u = 0; u < kLanes; u++) acc[u] = 0.f;
  int i = slice;
  for (; i + (kLanes - 1) * kSlices < n; i += kLanes * kSlices) {
    float v[kLanes];
#pragma unroll
    for (int u = 0; u < kLanes; u++) v[u] = part[(int64_t)(i + u * kSlices) * kHeadDim + d];
#pragma unroll
    for (int u = 0; u < kLanes; u++) acc[u] += v[u];
  }
  for (int u = 0; i < n; i += kSlices, u++) acc[u] += part[(int64_t)i * kHeadDim + d];
#pragma unroll
  for (int w = kLanes / 2; w > 0; w /= 2)
#pragma unroll
    for (int u = 0; u < w; u++) acc[u] += acc[u + w];
  red[slice][d] = acc[0];
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kSlices; k++) sum += red[k][d];
    (kmode ? a.dkw : a.dqw)[d] = sum;
  }
}

}  // namespace

hipError_t launch_bwd_dw_zero(float* dqw, float* dkw, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dw_zero_kernel, dim3(1), dim3(kHeadDim), 0, st, dqw, dkw);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(a.Sp / kPrepTok, a.B * (a.Hq + a.Hkv)), dim3(256), 0, st, a);
  return hipGetLastError();
}

int bwd_k_blocks(int32_t S, int32_t window) { return window > 0 ? (S + 127) / 128 : (S + kKvfKeys - 1) / kKvfKeys; }

hipError_t launch_bwd_kv(const BwdArgs& a, hipStream_t st) {
  // causal layers: dK and dV in one kernel, key blocks paired (two per work-group, the middle one alone when their
  // count is odd)
  if (a.window == 0) {
    const int nkb = bwd_k_blocks(a.S, 0);
    hipLaunchKernelGGL(bwd_kvf_kernel, dim3(a.B * a.Hkv * ((nkb + 1) / 2)), dim3(512), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(a.B * a.Hkv * bwd_k_blocks(a.S, a.window));
  hipLaunchKernelGGL(bwd_kv_kernel<false>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_kv_kernel<true>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_q(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_q_kernel, dim3(a.B * a.Hkv * ((a.S + kT - 1) / kT)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dw_reduce(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dw_reduce_kernel, dim3(2), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace zg
