// MiniMax-M3 block-sparse selection (ferrox_core block_sparse.rs on
// docs.rs, ferrox-core 0.14.0: module docs "Four rules", the public
// selection entry's doc comment, and the per-head selection's comments on
// scoring by the best position and on ties toward the lower block).
//
// Pass 1 (block_max): a block's score for (query, KV head) is the MAX over
// the block's causally visible positions of the page's f32 dot - products
// rounded to f32 and added in index order from +0, never fused.  That order
// is part of the definition, so the dots run on the VALU with contraction
// off; each lane owns one position and carries RC row accumulators
// (row = query x head of the workgroup's query tile), the query values are
// wave-uniform, the block's keys are staged in LDS in 32-wide d chunks.
// Pass 2 (select): per (query, head), force the init/local blocks, radix
// select the best budget - #forced of the others by (score desc, block asc),
// and write the union ascending.
#include "si_internal.hpp"

#pragma clang fp contract(off)

namespace si {

constexpr int kBlkThreads = 128;  // lanes = positions of one block pass
constexpr int kBlkRows = 32;      // accumulator rows per lane
constexpr int kBlkDChunk = 32;

__device__ __forceinline__ int64_t n_blocks_of(int64_t pos, int64_t n_pos, int bs) {
  if (pos < 0) return 0;
  int64_t nb = pos / bs + 1;
  int64_t ex = (n_pos + bs - 1) / bs;
  return nb < ex ? nb : ex;
}

struct BlockArgs {
  const float* q;
  const float* k;
  const int64_t* qpos;
  int32_t n_q, H, D;
  int64_t n_pos;
  int32_t bs, top, init, local;
  int32_t* out;
  int32_t width;
  int32_t* count;
  float* bscore;  // [n_q, H, max_blocks]
  int64_t max_blocks;
  int32_t qt;     // queries per tile (rows per tile = qt * H)
};

__global__ __launch_bounds__(kBlkThreads) void block_max(BlockArgs a) {
  __shared__ float ks[kBlkThreads][kBlkDChunk + 1];
  __shared__ float red[kBlkThreads / 64][kBlkRows];
  const int64_t lin = blockIdx.x;
  const int64_t b = lin % a.max_blocks;
  const int tile = (int)(lin / a.max_blocks);
  const int q0 = tile * a.qt;
  const int rows = a.qt * a.H;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

  // furthest position any query of the tile may see in this block
  int64_t maxpos = -1;
  for (int i = 0; i < a.qt && q0 + i < a.n_q; ++i) {
    int64_t p = a.qpos[q0 + i];
    if (b < n_blocks_of(p, a.n_pos, a.bs) && p > maxpos) maxpos = p;
  }
  if (maxpos < 0) return;
  const int64_t blk_lo = b * a.bs;
  int64_t blk_hi = blk_lo + a.bs;
  if (blk_hi > a.n_pos) blk_hi = a.n_pos;
  if (blk_hi > maxpos + 1) blk_hi = maxpos + 1;

  for (int r0 = 0; r0 < rows; r0 += kBlkRows) {
    float best[kBlkRows];
#pragma unroll
    for (int i = 0; i < kBlkRows; ++i) best[i] = -__builtin_inff();
    for (int64_t p0 = blk_lo; p0 < blk_hi; p0 += kBlkThreads) {
      const int64_t p = p0 + t;
      float acc[kBlkRows];
#pragma unroll
      for (int i = 0; i < kBlkRows; ++i) acc[i] = 0.0f;  // +0 start
      for (int dc = 0; dc < a.D; dc += kBlkDChunk) {
        const int dn = (a.D - dc) < kBlkDChunk ? (a.D - dc) : kBlkDChunk;
        __syncthreads();
        for (int e = t; e < kBlkThreads * kBlkDChunk; e += kBlkThreads) {
          int pr = e / kBlkDChunk, c = e % kBlkDChunk;
          int64_t pp = p0 + pr;
          ks[pr][c] = (pp < blk_hi && c < dn) ? a.k[pp * a.D + dc + c] : 0.0f;
        }
        __syncthreads();
        for (int c = 0; c < dn; ++c) {
          const float kd = ks[t][c];
#pragma unroll
          for (int i = 0; i < kBlkRows; ++i) {
            const int row = r0 + i;
            const int qi = row / a.H, h = row - qi * a.H;
            const int qq = q0 + qi;
            float qv = 0.0f;
            if (row < rows && qq < a.n_q) qv = a.q[((int64_t)qq * a.H + h) * a.D + dc + c];
            const float prod = qv * kd;
            acc[i] = acc[i] + prod;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kBlkRows; ++i) {
        const int row = r0 + i;
        const int qq = q0 + row / a.H;
        bool vis = p < blk_hi && row < rows && qq < a.n_q && p <= a.qpos[qq];
        if (vis && acc[i] > best[i]) best[i] = acc[i];
      }
    }
    // max over the block's positions (exact in any order)
#pragma unroll
    for (int i = 0; i < kBlkRows; ++i) {
      float v = best[i];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
      if (lane == 0) red[wv][i] = v;
    }
    __syncthreads();
    if (t < kBlkRows) {
      const int row = r0 + t;
      const int qi = row / a.H, h = row - qi * a.H;
      const int qq = q0 + qi;
      if (row < rows && qq < a.n_q && b < n_blocks_of(a.qpos[qq], a.n_pos, a.bs)) {
        float v = red[0][t];
        for (int w2 = 1; w2 < kBlkThreads / 64; ++w2) v = __builtin_fmaxf(v, red[w2][t]);
        a.bscore[((int64_t)qq * a.H + h) * a.max_blocks + b] = v;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// block_max for 128-position blocks and D <= 128 (the MiniMax-M3 shape):
// register-tiled VALU dots.  A workgroup owns a tile of 64 rows (flattened
// (query, head) pairs) and a run of kBmRun blocks.  The tile's q sits in
// LDS transposed [d][row]; each block's keys are staged 16 d at a time,
// transposed [d][position].  Thread t computes rows 8 (t / 32) .. +7 for
// positions 4 (t % 32) .. +3 of the block: per d step three 16-byte LDS
// reads feed 32 separately rounded products and 32 adds, in d order from +0
// exactly as the scalar definition.  Block maxima: over the thread's 4
// positions, then across the 32 lanes sharing the rows; lane j of those 32
// keeps the maxima of the run's block j and the run's maxima leave as one
// 128-byte row segment per row.
// Workgroup order: workgroups go to the 8 XCDs round robin, so workgroup b
// runs on XCD b % 8.  Each XCD takes every tile for one run after another
// (runs x, 15 - x, 16 + x, 31 - x, ... for XCD x: equal causal work per
// XCD), so the workgroups resident on an XCD share one run's keys (2 MB at
// D 128) in its L2 and the keys come from HBM about once.
// ---------------------------------------------------------------------------
constexpr int kBmRows = 64;
constexpr int kBmPos = 128;
constexpr int kBmDC = 16;
constexpr int kBmMaxD = 128;
constexpr int kBmRun = 32;  // blocks per workgroup

__global__ __launch_bounds__(256) void block_max128(BlockArgs a, int runs, int64_t tiles) {
  __shared__ __attribute__((aligned(16))) float qs[kBmMaxD][kBmRows];
  __shared__ __attribute__((aligned(16))) float ks[2][kBmDC][kBmPos];
  __shared__ int64_t rpos[kBmRows];
  __shared__ int64_t tile_blocks;
  const int t = threadIdx.x;
  const int xcd = (int)(blockIdx.x % 8);
  const int64_t seq = blockIdx.x / 8;
  const int64_t slot = seq / tiles, tile = seq % tiles;
  const int run = (int)(8 * slot + ((slot & 1) ? 7 - xcd : xcd));
  if (run >= runs) return;  // padding of the run count to a multiple of 8
  const int64_t nrows = (int64_t)a.n_q * a.H;
  const int64_t row0 = (int64_t)tile * kBmRows;
  const int D = a.D;
  if (t == 0) tile_blocks = 0;
  __syncthreads();
  if (t < kBmRows) {
    const int64_t row = row0 + t;
    int64_t p = -1;
    if (row < nrows) p = a.qpos[row / a.H];
    rpos[t] = p;
    const int64_t nb = n_blocks_of(p, a.n_pos, a.bs);
    atomicMax(reinterpret_cast<unsigned long long*>(&tile_blocks), (unsigned long long)nb);
  }
  __syncthreads();
  const int64_t b_lo = (int64_t)run * kBmRun;
  const int64_t b_hi = tile_blocks < b_lo + kBmRun ? tile_blocks : b_lo + kBmRun;
  if (b_lo >= b_hi) return;  // uniform: no row of the tile sees these blocks
  // q tile, transposed
  for (int e = t; e < kBmRows * D; e += 256) {
    const int row = e / D, d = e - row * D;
    const int64_t grow = row0 + row;
    qs[d][row] = grow < nrows ? a.q[grow * D + d] : 0.0f;
  }
  const int rg = t >> 5, pg = t & 31;
  int64_t myp[8], mynb[8];  // the rows' query positions and visible block counts
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    myp[i] = rpos[8 * rg + i];
    mynb[i] = n_blocks_of(myp[i], a.n_pos, a.bs);
  }
  const int nchunk = (D + kBmDC - 1) / kBmDC;
  // key staging: thread t loads position t / 2, d's (t & 1) * 8 .. +7 of the chunk
  const int sp = t >> 1, sd = (t & 1) * 8;
  // lane pg keeps the maxima of the run's block b_lo + pg for its 8 rows
  float keep[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) keep[i] = -__builtin_inff();
  // fetch a chunk into registers before the compute, write it to LDS after
  float kr[8];
  auto fetch = [&](int64_t b, int c) {
    const int64_t pos = b * kBmPos + sp;
    const int d0 = c * kBmDC + sd;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = d0 + j;
      kr[j] = (pos < a.n_pos && d < D) ? a.k[pos * D + d] : 0.0f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) ks[buf][sd + j][sp] = kr[j];
  };
  __syncthreads();
  for (int64_t b = b_lo; b < b_hi; ++b) {
    float acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;  // +0 start
    fetch(b, 0);
    stash(0);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
      const int buf = c & 1;
      if (c + 1 < nchunk) fetch(b, c + 1);
      const int dn = (D - c * kBmDC) < kBmDC ? (D - c * kBmDC) : kBmDC;
      auto dstep = [&](int dd) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[c * kBmDC + dd][8 * rg]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[c * kBmDC + dd][8 * rg + 4]);
        const float4 kv = *reinterpret_cast<const float4*>(&ks[buf][dd][4 * pg]);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float prod = qv[i] * kk[j];
            acc[i][j] = acc[i][j] + prod;
          }
      };
      if (dn == kBmDC) {  // whole chunk: unrolled, so the LDS reads run ahead
#pragma unroll
        for (int dd = 0; dd < kBmDC; ++dd) dstep(dd);
      } else {
        for (int dd = 0; dd < dn; ++dd) dstep(dd);
      }
      // buffer buf ^ 1 was last read in chunk c - 1, before the previous barrier
      if (c + 1 < nchunk) stash(buf ^ 1);
      __syncthreads();
    }
    // block maxima over the visible positions (max is exact in any order)
    const int64_t pos0 = b * kBmPos + 4 * pg;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float m = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t pos = pos0 + j;
        if (pos < a.n_pos && pos <= myp[i] && acc[i][j] > m) m = acc[i][j];
      }
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
      keep[i] = pg == (int)(b - b_lo) ? m : keep[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = row0 + 8 * rg + i;
    const int64_t b = b_lo + pg;
    if (row < nrows && b < b_hi && b < mynb[i]) a.bscore[row * a.max_blocks + b] = keep[i];
  }
}

constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void block_select(BlockArgs a) {
  __shared__ int hist[2048];
  __shared__ int red[kSelThreads / 64 + 4];
  __shared__ uint64_t list[kMaxTopk];
  __shared__ int counter;
  const int qq = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int64_t n = n_blocks_of(a.qpos[qq], a.n_pos, a.bs);
  int32_t* out = a.out + (int64_t)blockIdx.x * a.width;
  const int64_t fi = a.init < n ? a.init : n;
  const int64_t ls = n - (a.local < n ? a.local : n);  // first local block
  const int64_t lo_end = fi, hi_beg = ls > fi ? ls : fi;
  const int64_t nf = lo_end + (n - hi_beg);
  const int64_t budget = a.top > nf ? a.top : nf;
  int64_t total;  // blocks written
  if (threadIdx.x == 0) counter = 0;
  __syncthreads();
  if (n == 0) {
    total = 0;
  } else if (nf >= budget || nf == n) {
    for (int64_t i = threadIdx.x; i < nf; i += kSelThreads)
      out[i] = (int32_t)(i < lo_end ? i : hi_beg + (i - lo_end));
    total = nf;
  } else {
    const int64_t m = hi_beg - lo_end;  // scored blocks [fi, ls)
    const int64_t take = (budget - nf) < m ? (budget - nf) : m;
    if (take == m) {
      for (int64_t i = threadIdx.x; i < n; i += kSelThreads) out[i] = (int32_t)i;
      total = n;
    } else {
      const float* sc = a.bscore + (int64_t)blockIdx.x * a.max_blocks + lo_end;
      auto load = [&](int64_t i) -> uint32_t { return order_key(sc[i]); };
      int64_t n_gt;
      const uint32_t thr = radix_select_kth<kSelThreads>(load, m, take, hist, red, &n_gt);
      // forced blocks first, then the chosen ones; values are ~block so a
      // descending sort gives ascending blocks
      for (int64_t i = threadIdx.x; i < nf; i += kSelThreads) {
        int64_t blk = i < lo_end ? i : hi_beg + (i - lo_end);
        list[i] = (uint64_t)(0xFFFFFFFFu - (uint32_t)blk);
      }
      for (int64_t i = threadIdx.x; i < m; i += kSelThreads)
        if (load(i) > thr)
          list[nf + atomicAdd(&counter, 1)] = (uint64_t)(0xFFFFFFFFu - (uint32_t)(lo_end + i));
      const int need = (int)(take - n_gt);
      int taken = 0;
      for (int64_t base = 0; base < m && taken < need; base += kSelThreads) {
        int64_t i = base + threadIdx.x;
        int flag = (i < m && load(i) == thr) ? 1 : 0;
        int tot;
        int rank = block_excl_scan<kSelThreads>(flag, red, &tot);
        if (flag && taken + rank < need)
          list[nf + n_gt + taken + rank] = (uint64_t)(0xFFFFFFFFu - (uint32_t)(lo_end + i));
        taken += tot;
      }
      total = nf + take;
      const int P = next_pow2((int)total);
      for (int i = (int)total + threadIdx.x; i < P; i += kSelThreads) list[i] = 0ull;
      __syncthreads();
      bitonic_sort_desc<kSelThreads>(list, P);
      for (int64_t i = threadIdx.x; i < total; i += kSelThreads)
        out[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)list[i]);
    }
  }
  for (int64_t i = total + threadIdx.x; i < a.width; i += kSelThreads) out[i] = -1;
  if (a.count && threadIdx.x == 0) a.count[blockIdx.x] = (int32_t)total;
}

}  // namespace si

extern "C" size_t block_sparse_select_workspace(int32_t n_q, int32_t n_kv_heads, int64_t n_pos,
                                                int32_t block_size) {
  if (n_q <= 0 || n_kv_heads <= 0 || n_pos <= 0 || block_size <= 0) return 0;
  const int64_t mb = (n_pos + block_size - 1) / block_size;
  return (size_t)n_q * (size_t)n_kv_heads * (size_t)mb * sizeof(float);
}

namespace si {
hipError_t launch_block_select(const float* q, const float* k, const int64_t* qpos, int32_t n_q,
                               int32_t H, int32_t D, int64_t n_pos, int32_t bs, int32_t top,
                               int32_t init, int32_t local, int32_t* out, int32_t width,
                               int32_t* count, float* ws, hipStream_t st) {
  BlockArgs a;
  a.q = q; a.k = k; a.qpos = qpos; a.n_q = n_q; a.H = H; a.D = D; a.n_pos = n_pos;
  a.bs = bs; a.top = top; a.init = init; a.local = local; a.out = out; a.width = width;
  a.count = count; a.bscore = ws;
  a.max_blocks = (n_pos + bs - 1) / bs;
  a.qt = H >= kBlkRows ? 1 : kBlkRows / H;
  if (n_q == 0) return hipSuccess;
  if (bs == kBmPos && D <= kBmMaxD && a.max_blocks > 0) {
    const int64_t tiles = ((int64_t)n_q * H + kBmRows - 1) / kBmRows;
    const int runs = (int)((a.max_blocks + kBmRun - 1) / kBmRun);
    const int64_t runs8 = (runs + 7) / 8 * 8;
    hipLaunchKernelGGL(block_max128, dim3((unsigned)(tiles * runs8)), dim3(256), 0, st, a, runs,
                       tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const int64_t tiles = (n_q + a.qt - 1) / a.qt;
    if (tiles * a.max_blocks > 0) {
      hipLaunchKernelGGL(block_max, dim3((unsigned)(tiles * a.max_blocks)), dim3(kBlkThreads), 0,
                         st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(block_select, dim3((unsigned)((int64_t)n_q * H)), dim3(kSelThreads), 0, st,
                     a);
  return hipGetLastError();
}
}  // namespace si
