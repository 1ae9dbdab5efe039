// Sparse MLA decode attention over the rows a swap call returned.
//
// "SGLang HiSparse" blog, section 1 (attention is exact over the positions
// the indexer selected) and section 2.1 (the sparse table a swap-in returns
// goes straight to decode attention).  Absorbed-MLA decode form: each KV row
// holds a 512-dim latent c and a 64-dim rope key r; for head h
//   s_i = scale * (q_h[:512].c_i + q_h[512:].r_i),  out_h = softmax(s) . c,
//   lse_h = log sum exp(s).
//
// Work split: one workgroup = 4 waves = 64 heads of one batch row over one
// range of its locations (split-K over locations when the batch is small;
// a second kernel merges the splits by their log-sum-exp).  Tiles of 32 rows
// are gathered into LDS as bf16 (fp8 rows are dequantised on the way).  Each
// wave owns 16 heads and computes with MFMA 16x16x32 bf16:
//   S^T (tokens x heads) = K (tokens x 576) . Q^T   -- Q^T lives in registers
//   O^T (dims x heads)  += V^T (dims x tokens) . P^T
// With heads as the N dimension every lane's accumulators belong to one head,
// so the online-softmax rescale is a per-lane scalar, and the C layout of S^T
// is directly the B operand of the P.V product (the 8 tokens a lane holds
// are used as its 8 k-slots, and V^T is read with the same token order).
#include "internal.h"

namespace hisparse {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;     // 576
constexpr int kTile = 32;                 // rows per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;  // 256
constexpr int kHeadsPerGroup = 16 * kWaves;
constexpr int kRowElems = kDim + 16;      // LDS row pitch in bf16 (1184 B)
constexpr int kKSteps = kDim / 32;        // 18
constexpr float kLn2 = 0.69314718055994530942f;

struct MlaArgs {
  const uint16_t* q;          // bf16 bits [B][Hq][576]
  const int32_t* locs;        // [B][n_locs]
  const int32_t* page_table;  // [B][pt_stride] or null (token rows)
  const uint8_t* kv;          // the layer's hot buffer
  int64_t kv_rows;            // token rows in kv
  int32_t item_bytes;         // 1152 (bf16) or 656 (fp8)
  int32_t page_size;
  int32_t pt_stride;
  int32_t batch, heads, n_locs, splits, per_split, groups, units;
  float scale_log2;           // softmax scale * log2(e)
  float* out;                 // [B][Hq][512]
  float* lse;                 // [B][Hq] or null
  float* part_out;            // [B][splits][Hq][512]
  float* part_ml;             // [B][splits][Hq][2]: running max (log2 units), sum
  uint32_t* err;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Token row of location `loc` of batch row b, or -1.
__device__ __forceinline__ int64_t token_row(const MlaArgs& a, int b, int32_t loc) {
  if (loc < 0) return -1;
  int64_t row;
  if (a.page_table == nullptr) {
    row = loc;
  } else {
    const int j = loc / a.page_size;
    if (j >= a.pt_stride) return -1;
    const int32_t page = a.page_table[static_cast<size_t>(b) * a.pt_stride + j];
    if (page < 0) return -1;
    row = static_cast<int64_t>(page) * a.page_size + (loc - j * a.page_size);
  }
  return row < a.kv_rows ? row : -1;
}

// Gathers rows [t0, t0 + kTile) of batch row b into the LDS tile as bf16.
__device__ void load_tile(const MlaArgs& a, int b, int t0, int t_end, uint16_t* tile,
                          int* tvalid) {
  const int tid = threadIdx.x;
  __shared__ int64_t s_row[kTile];
  if (tid < kTile) {
    const int t = t0 + tid;
    int64_t row = -1;
    if (t < t_end) {
      row = token_row(a, b, a.locs[static_cast<size_t>(b) * a.n_locs + t]);
      if (row < 0 && a.locs[static_cast<size_t>(b) * a.n_locs + t] >= 0)
        raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
    }
    s_row[tid] = row;
    tvalid[tid] = row >= 0;
  }
  __syncthreads();
  if (a.item_bytes == 2 * kDim) {
    // bf16 rows: 72 chunks of 16 bytes each
    for (int c = tid; c < kTile * 72; c += kThreads) {
      const int r = c / 72, col = c - r * 72;
      const int64_t row = s_row[r];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row >= 0)
        v = *reinterpret_cast<const u32x4*>(a.kv + row * a.item_bytes + col * 16);
      *reinterpret_cast<u32x4*>(tile + r * kRowElems + col * 8) = v;
    }
  } else {
    // fp8 rows: 32 latent chunks of 16 codes (dequantised with their tile's
    // scale) and 8 rope chunks of 8 bf16
    for (int c = tid; c < kTile * 40; c += kThreads) {
      const int r = c / 40, col = c - r * 40;
      const int64_t row = s_row[r];
      const uint8_t* src = a.kv + row * a.item_bytes;
      if (col < 32) {
        u16x8 lo = {0, 0, 0, 0, 0, 0, 0, 0}, hi = lo;
        if (row >= 0) {
          const u32x4 codes = *reinterpret_cast<const u32x4*>(src + col * 16);
          const float scale = *reinterpret_cast<const float*>(src + kLatent + (col >> 3) * 4);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x2 x0 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], false);
            const f32x2 x1 = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], true);
            const uint16_t e0 = bf16_bits(x0[0] * scale), e1 = bf16_bits(x0[1] * scale);
            const uint16_t e2 = bf16_bits(x1[0] * scale), e3 = bf16_bits(x1[1] * scale);
            if (w < 2) {
              lo[4 * w] = e0; lo[4 * w + 1] = e1; lo[4 * w + 2] = e2; lo[4 * w + 3] = e3;
            } else {
              hi[4 * (w - 2)] = e0; hi[4 * (w - 2) + 1] = e1;
              hi[4 * (w - 2) + 2] = e2; hi[4 * (w - 2) + 3] = e3;
            }
          }
        }
        *reinterpret_cast<u16x8*>(tile + r * kRowElems + col * 16) = lo;
        *reinterpret_cast<u16x8*>(tile + r * kRowElems + col * 16 + 8) = hi;
      } else {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row >= 0)
          v = *reinterpret_cast<const u32x4*>(src + kLatent + 16 + (col - 32) * 16);
        *reinterpret_cast<u32x4*>(tile + r * kRowElems + kLatent + (col - 32) * 8) = v;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void mla_decode(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * kRowElems];
  __shared__ int tvalid[kTile];

  // XCD-aware mapping: the head groups of one (row, split) unit run on the
  // same XCD (workgroups are dealt to the 8 XCDs round robin) and share its
  // rows through that XCD's L2.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int k = id >> 3;
  const int hg = k % a.groups;
  const int unit = (k / a.groups) * 8 + xcd;
  if (unit >= a.units) return;
  const int b = unit / a.splits;
  const int split = unit - b * a.splits;
  const int t_begin = split * a.per_split;
  const int t_end = min(a.n_locs, t_begin + a.per_split);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;       // lane group
  const int n = lane & 15;       // head within the wave / row within a 16-tile
  const int head = hg * kHeadsPerGroup + wave * 16 + n;
  const bool head_ok = head < a.heads;

  // Q^T operand: lane holds q[head][32*ks + 8*g .. +8] for every k-step
  bf16x8 qreg[kKSteps];
  {
    const uint16_t* qh = a.q + (static_cast<size_t>(b) * a.heads + (head_ok ? head : 0)) * kDim;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qh + 32 * ks + 8 * g);
      if (!head_ok) v = u32x4{0u, 0u, 0u, 0u};
      qreg[ks] = as_bf16x8(v);
    }
  }
  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // running sum of exp2(score - m_run)

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    load_tile(a, b, t0, t_end, tile, tvalid);
    __syncthreads();

    // S^T for tokens [0,16) and [16,32) of the tile
    f32x4 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = tile + (st * 16 + n) * kRowElems + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const bf16x8 kv = as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32 * ks));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qreg[ks], c, 0, 0, 0);
      }
      s[st] = c;
    }
    // online softmax for this lane's head; lane holds tokens 4g+i and 16+4g+i
    float sc[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
      const float v = tvalid[tok] ? s[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
      sc[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    u16x8 pbits;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = m_new == -INFINITY ? 0.f : exp2f(sc[i] - m_new);
      const uint16_t pb = bf16_bits(p);
      pbits[i] = pb;
      psum += __builtin_bit_cast(float, static_cast<uint32_t>(pb) << 16);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    const bf16x8 pop = __builtin_bit_cast(bf16x8, pbits);

    // O^T += V^T . P^T; quad u covers dims 64u .. 64u+63, lane row n <-> dims
    // 64u + 4n + j for the four sub-tiles j
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      u16x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tok = (i < 4 ? 0 : 16) + 4 * g + (i & 3);
        v[i] = *reinterpret_cast<const u16x4*>(tile + tok * kRowElems + 64 * u + 4 * n);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u16x8 col;
#pragma unroll
        for (int i = 0; i < 8; ++i) col[i] = v[i][j];
        acc[4 * u + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, col), pop, acc[4 * u + j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (!head_ok) return;
  // lane holds head `head`, dims 64u + 16g + 4i + j  (sub-tile (u, j), C row 4g + i)
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* dst;
  if (a.splits == 1) {
    dst = a.out + (static_cast<size_t>(b) * a.heads + head) * kLatent;
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<size_t>(b) * a.heads + head] =
          l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const size_t ps = (static_cast<size_t>(b) * a.splits + split) * a.heads + head;
    dst = a.part_out + ps * kLatent;
    if (g == 0) {
      a.part_ml[2 * ps] = m_run;
      a.part_ml[2 * ps + 1] = l_run;
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 o = {acc[4 * u][i] * inv, acc[4 * u + 1][i] * inv, acc[4 * u + 2][i] * inv,
                 acc[4 * u + 3][i] * inv};
      *reinterpret_cast<f32x4*>(dst + 64 * u + 16 * g + 4 * i) = o;
    }
  }
}

// Merges the splits of every (row, head) by their log-sum-exp.
__global__ __launch_bounds__(128) void mla_combine(MlaArgs a) {
  const int bh = blockIdx.x;  // b * heads + h
  const int b = bh / a.heads, h = bh - b * a.heads;
  float big = -INFINITY;
  for (int s = 0; s < a.splits; ++s) {
    const size_t ps = (static_cast<size_t>(b) * a.splits + s) * a.heads + h;
    const float l = a.part_ml[2 * ps + 1];
    if (l > 0.f) big = fmaxf(big, a.part_ml[2 * ps] + log2f(l));
  }
  float wsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
    const size_t ps = (static_cast<size_t>(b) * a.splits + s) * a.heads + h;
    const float l = a.part_ml[2 * ps + 1];
    if (!(l > 0.f)) continue;
    const float w = exp2f(a.part_ml[2 * ps] + log2f(l) - big);
    wsum += w;
    const f32x4 p = *reinterpret_cast<const f32x4*>(a.part_out + ps * kLatent + 4 * threadIdx.x);
    o += w * p;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<f32x4*>(a.out + static_cast<size_t>(bh) * kLatent + 4 * threadIdx.x) = o * inv;
  if (a.lse != nullptr && threadIdx.x == 0)
    a.lse[bh] = wsum > 0.f ? (big + log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

// Splits of the location list per batch row: enough workgroups to cover the
// CUs twice, at least 128 locations per split.
int mla_splits(int batch, int heads, int n_locs, int num_cus) {
  const int groups = (heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int units = batch * groups;
  int splits = (2 * num_cus + units - 1) / units;
  splits = min(splits, max(1, n_locs / 128));
  return max(1, min(splits, 64));
}

size_t mla_workspace_bytes(int batch, int heads, int n_locs, int num_cus) {
  const int splits = mla_splits(batch, heads, n_locs, num_cus);
  if (splits == 1) return 0;
  return static_cast<size_t>(batch) * splits * heads * (kLatent + 2) * sizeof(float);
}

hipError_t launch_mla_decode(const MlaDecodeCall& c, hipStream_t s) {
  MlaArgs a{};
  a.q = static_cast<const uint16_t*>(c.q);
  a.locs = c.locs;
  a.page_table = c.page_table;
  a.kv = c.kv;
  a.kv_rows = c.kv_rows;
  a.item_bytes = c.item_bytes;
  a.page_size = c.page_size;
  a.pt_stride = c.pt_stride;
  a.batch = c.batch;
  a.heads = c.heads;
  a.n_locs = c.n_locs;
  a.splits = mla_splits(c.batch, c.heads, c.n_locs, c.num_cus);
  a.per_split = ((c.n_locs + a.splits - 1) / a.splits + kTile - 1) / kTile * kTile;
  a.groups = (c.heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  a.units = c.batch * a.splits;
  a.scale_log2 = c.scale * 1.44269504088896340736f;
  a.out = c.out;
  a.lse = c.lse;
  a.err = c.err;
  if (a.splits > 1) {
    a.part_out = static_cast<float*>(c.workspace);
    a.part_ml = a.part_out + static_cast<size_t>(c.batch) * a.splits * c.heads * kLatent;
  }
  const int padded_units = (a.units + 7) / 8 * 8;
  hipLaunchKernelGGL(mla_decode, dim3(padded_units * a.groups), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(mla_combine, dim3(c.batch * c.heads), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace hisparse
