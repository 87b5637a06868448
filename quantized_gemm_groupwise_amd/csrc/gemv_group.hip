// Grouped decode (M <= 4): many linears in one call, over a device plan of
// their row tiles sorted into kernel classes.  The per-tile arithmetic is
// the single-linear kernel's (gemv_core.h), so each output is the same
// bits as one gq_linear call.
#include <string.h>

#include <mutex>

#include "gemv_core.h"

namespace gq {
namespace {

// The wave's R * M sums reduced across lanes; one lane per output stores
// y[m][n0 + r] (row stride N) for n0 + r < nlim.
template <int ACT, int M, int R, int BITS>
__device__ __forceinline__ void reduce_store(const float (&acc)[R][M], int lane, int n0, int nlim,
                                             int N, uint16_t *y) {
  if constexpr (mfma_decode(BITS, M, R)) {
    mfma_reduce_store<ACT, M>(acc[0], lane, n0, nlim, N, y);
    return;
  }
  constexpr int V0 = R * M;
  constexpr int V = V0 <= 1 ? 1 : V0 <= 2 ? 2 : V0 <= 4 ? 4 : V0 <= 8 ? 8 : 16;
  float vals[V];
#pragma unroll
  for (int v = 0; v < V; ++v) vals[v] = v < V0 ? acc[v / M][v % M] : 0.f;
  const float tot = wave_reduce_multi<V>(vals, lane);
  const int idx = reduced_index<V>(lane);
  if ((lane & ((64 / V) - 1)) == 0 && idx < V0) {
    const int r = idx / M, m = idx % M;
    if (n0 + r < nlim)
      store_global16(y, (int64_t)m * N + n0 + r, ACT == 0 ? f32_to_bf16_rne(tot) : f32_to_f16_bits(tot));
  }
}

// Position in a class's tile list: segment si, tile t of that segment; T is
// the class tile index, [T0, T1) the workgroup's current chunk.
struct TilePos {
  int si, t, T, T0, T1;
};

// Grouped decode: workgroup w of G of one class of a plan.  Every tile runs
// the single-linear kernel's arithmetic and order, so the outputs are the
// same bits as one gq_linear call per linear.  x of a linear is staged once per workgroup
// while consecutive tiles stay in that linear.  Every branch below depends
// only on the workgroup and the plan, so the waves of a workgroup meet the
// same barriers.
//
// PIPE (persistent launch; every row fits one load group and one staged
// chunk): workgroup w of G takes the contiguous tile range of its share of
// the class's bytes and walks it segment by segment, software pipelined --
// each wave issues the loads of its next tile before it works on the
// current one, so two tiles of codes are in flight per wave.  Segment data
// is read once per segment and a tile's row resources are a multiply-add
// from the segment's base addresses.  The pipeline restarts where the
// linear changes (x must be restaged first).
//
// Otherwise workgroup w takes the class's chunks of `chunk` tiles
// w, w + G, ... (a grid of one workgroup per tile when chunk is 1 and G the
// tile count) and runs each tile with the single-linear kernel's workgroup
// body (rows in one load group when ONE, else streamed group by group).
template <int ACT, int M, int BITS, int SS, int NL, bool ONE, bool PIPE>
__device__ __forceinline__ void group_body(const uint8_t *__restrict__ plan, int cls, int chunk,
                                           const int G, const int w, uint32_t *lds) {
  constexpr int R = group_r(BITS, M);
  constexpr int kTile = group_tile(BITS, M);
  using Gm = Geo<BITS>;
  if constexpr (chunk_slices(BITS, M, SS) < 1) {
    return;                                 // never launched: SS too small for M
  } else {
  const GroupPlanHeader &H = *reinterpret_cast<const GroupPlanHeader *>(plan);
  const GroupClass &C = H.cls[cls];
  const GroupSeg *segs = reinterpret_cast<const GroupSeg *>(plan + H.segs_off) + C.seg0;
  const GroupItemDev *items = reinterpret_cast<const GroupItemDev *>(plan + H.items_off);
  const int nseg = C.nseg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int lane = threadIdx.x & (kLanes - 1);

  if constexpr (ONE && PIPE) {
    // byte range [lo, hi) of the class; the tiles whose first byte is in it
    const int64_t lo = C.bytes * w / G, hi = C.bytes * (w + 1) / G;
    int ls = 0;
    {
      int a = 0, b = nseg - 1;              // last segment starting at or before lo
      while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if (segs[mid].cbyte0 <= lo) a = mid;
        else b = mid - 1;
      }
      ls = a;
    }
    int lt = (int)((lo - segs[ls].cbyte0 + segs[ls].tile_bytes - 1) / segs[ls].tile_bytes);
    if (lt >= segs[ls].ntiles) {
      if (++ls >= nseg) return;
      lt = 0;
    }
    // Load cursor: the tile whose loads are issued next.  Its segment's
    // fields are read from the plan once per segment and kept in scalar
    // registers (stores through y could alias the plan, so fields read
    // again after a store would be loaded again); within a segment the
    // cursor steps by one tile with a few adds.
    int64_t lcb;                            // class byte of the cursor's tile
    int64_t ltb;                            // bytes per tile of its segment
    int lend;                               // tiles of the segment
    int litem;                              // its linear
    const uint8_t *pc;                      // codes of the wave's first row in the tile
    const uint16_t *ps;                     // its scales
    const uint8_t *pz;                      // its zero points
    int lrows;                              // rows of the run from that row on
    int ln0, lnlim;                         // that row in the linear; end of the run
    int K = 0;                              // K of the linear being worked on
    uint32_t RB = 0, GPR = 0;               // row bytes and groups per row
    auto open_seg = [&](int sg, int tt) {
      const GroupSeg &S = segs[sg];
      const int rw = tt * kTile + wave * R;
      lcb = S.cbyte0 + (int64_t)tt * S.tile_bytes;
      ltb = S.tile_bytes;
      lend = S.ntiles;
      litem = S.item;
      const int Ks = items[litem].L.K;
      const uint32_t rb = (uint32_t)(Ks * BITS / 8), gpr = (uint32_t)(Ks / Gm::G);
      pc = S.codes + (uint64_t)rw * rb;
      ps = S.scales + (uint64_t)rw * gpr;
      pz = S.zeros + (uint64_t)rw * gpr;
      lrows = S.rows - rw;
      ln0 = S.tile0 * kTile + rw;
      lnlim = S.tile0 * kTile + S.rows;
    };
    // step the cursor to the next tile of the range; false past its end
    auto advance = [&]() -> bool {
      if (++lt < lend) {
        lcb += ltb;
        pc += kTile * RB;
        ps += kTile * GPR;
        pz += kTile * GPR;
        lrows -= kTile;
        ln0 += kTile;
      } else {
        if (ls + 1 >= nseg) return false;
        ++ls;
        lt = 0;
        open_seg(ls, 0);
      }
      return lcb < hi;
    };
    // issue the loads of the cursor's tile into gl (or, when `none`, the
    // same number of loads of empty resources); rows past the run's end get
    // empty resources
    auto issue_cursor = [&](LoadGroup<BITS, R, NL> &gl, bool none) {
      RowRsrc<R> rr;
      if (!none) {
        make_row_rsrc<BITS, M, R>(rr, pc, ps, pz, RB, GPR, lrows);
      } else {
        rr.rb = rr.gpr = 0u;
#pragma unroll
        for (int r = 0; r < R; ++r) rr.c[r] = rr.s[r] = rr.z[r] = make_rsrc(plan, 0u);
      }
      issue_group<BITS, R, NL, false, mfma_decode(BITS, M, R)>(gl, 0, NL, lane, rr);
    };
    open_seg(ls, lt);
    if (lcb >= hi) return;

    uint4 *pairs = reinterpret_cast<uint4 *>(lds);
    int item = litem;
    const uint16_t *yp = nullptr;
    int yN = 0;
    auto stage = [&](int it) {
      const GroupItemDev &I = items[it];
      K = I.L.K;
      RB = (uint32_t)(K * BITS / 8);
      GPR = (uint32_t)(K / Gm::G);
      yp = reinterpret_cast<const uint16_t *>(I.y);
      yN = I.L.N;
      const int ns = (K * BITS / 8 + 1023) >> 10;
      const uint32_t xbytes = (uint32_t)(M * K) * 2u;
      StageRegs<SS> st;
      stage_x_load<BITS, M, SS>(st, make_rsrc(I.x, xbytes), xbytes, K, 0, ns);
      stage_x_store<BITS, ACT, M, SS>(st, ns, pairs,
                                      reinterpret_cast<float *>(lds + M * ns * Gm::PW * kLanes));
      lds_barrier();
    };
    // Work on the tile whose codes are in g (outputs from row n0, run end
    // nlim), after issuing the loads of the next tile of the same linear
    // into gn; returns false when the range is done.  The loads into gn are
    // issued on every path (with empty resources when there is no next tile
    // in this linear, so they return zeros without touching memory): the
    // wait before the work on g then counts only g's loads.
    int sn0 = 0, snlim = 0;                 // rows of the tile being worked on
    auto step = [&](LoadGroup<BITS, R, NL> &g, LoadGroup<BITS, R, NL> &gn) -> bool {
      const bool more = advance();
      const bool same = more && litem == item;
      issue_cursor(gn, !same);
      const int ns = (K * BITS / 8 + 1023) >> 10;
      const float *sm = reinterpret_cast<const float *>(lds + M * ns * Gm::PW * kLanes);
      float acc[R][M];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.f;
      compute_group<BITS, ACT, M, R, NL>(g, 0, ns, 0, lane, pairs, sm, ns, acc);
      // rows past the run (a partial last tile) are past N: not stored
      reduce_store<ACT, M, R, BITS>(acc, lane, sn0, snlim, yN, const_cast<uint16_t *>(yp));
      if (!more) return false;
      if (!same) {
        // the next tile is in another linear: restage x, then its loads
        item = litem;
        lds_barrier();
        stage(item);
        issue_cursor(gn, false);
      }
      sn0 = ln0;
      snlim = lnlim;
      return true;
    };
    stage(item);
    LoadGroup<BITS, R, NL> ga, gb;
    issue_cursor(ga, false);
    sn0 = ln0;
    snlim = lnlim;
    while (true) {
      if (!step(ga, gb)) break;
      if (!step(gb, ga)) break;
    }
  } else {
  const int tiles = C.tiles;
  // the segment holding class tile T
  auto seg_of_tile = [&](int T) -> int {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (segs[mid].ctile0 <= T) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  // chunks w, w + G, ... of `chunk` tiles
  if ((int64_t)w * chunk >= tiles) return;
  TilePos pos;
  pos.T0 = pos.T = w * chunk;
  pos.T1 = pos.T + chunk < tiles ? pos.T + chunk : tiles;
  pos.si = seg_of_tile(pos.T);
  pos.t = pos.T - segs[pos.si].ctile0;
  // normalize p (after p.t and p.T advanced by one) to a real tile, and say
  // whether the workgroup has one
  auto settle = [&](TilePos &p) -> bool {
    if (p.T >= p.T1) {                      // next chunk of this workgroup
      if ((int64_t)p.T0 + (int64_t)G * chunk >= tiles) return false;
      p.T0 = p.T = p.T0 + G * chunk;
      p.T1 = p.T + chunk < tiles ? p.T + chunk : tiles;
      p.si = seg_of_tile(p.T);
      p.t = p.T - segs[p.si].ctile0;
      return true;
    }
    while (p.t >= segs[p.si].ntiles) {
      ++p.si;
      p.t = 0;
    }
    return true;
  };
  int prev_item = -1;
  do {
    const int item = segs[pos.si].item;
    const GroupItemDev &I = items[item];
    const LayoutDev &L = I.L;
    const int nb = (segs[pos.si].tile0 + pos.t) * kTile;
    const int n0 = nb + wave * R;
    const int ns = (L.K * BITS / 8 + 1023) >> 10;
    // restage when the linear changes, or every tile when a row does not
    // fit one staged chunk; the barrier lets every wave finish reading
    // the previous x first
    const bool stage = item != prev_item || ns > chunk_slices(BITS, M, SS);
    if (stage && prev_item >= 0) lds_barrier();
    BlockInfo bi = {BITS, 0, 0};
    int blk = 0;
    if (!I.uniform) {
      blk = nb / L.block_n;
      bi = block_info(L, blk);
    }
    gemv_block<BITS, ACT, M, R, NL, SS, ONE>(
        L, bi, blk, n0, n0 < L.N, reinterpret_cast<const uint16_t *>(I.x),
        reinterpret_cast<const uint8_t *>(I.codes), reinterpret_cast<const uint16_t *>(I.scales),
        reinterpret_cast<const uint8_t *>(I.zeros), reinterpret_cast<uint16_t *>(I.y), lds, stage);
    prev_item = item;
    ++pos.t;
    ++pos.T;
  } while (settle(pos));
  }
  }
}

// One class of a plan per launch: the whole grid works on class `cls`.
template <int ACT, int M, int BITS, int SS, int NL, bool ONE, bool PIPE>
__global__ __launch_bounds__(kThreads) void gemv_group_kernel(const uint8_t *__restrict__ plan,
                                                              int cls, int chunk) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  group_body<ACT, M, BITS, SS, NL, ONE, PIPE>(plan, cls, chunk, gridDim.x, blockIdx.x, lds);
}

// Classes of one width that run one workgroup per tile, gathered into one
// launch: class j of the launch owns workgroups [start[j], start[j + 1]).
constexpr int kFuseMax = 9;                  // 3 staging x 3 load-group configurations
struct FuseArgs {
  int32_t n;                                 // classes in the launch
  int32_t cls[kFuseMax];                     // their indices in the plan
  int32_t one[kFuseMax];                     // their load-group configuration (GroupClass::one)
  int32_t start[kFuseMax + 1];               // first workgroup of each; start[n] = grid
};

// x staging sub-units per thread in the fused launch: the fewest whose
// staged chunk holds `slices` 1 KB slices.  Which thread stages which 16
// activations depends on this count, the LDS contents and the per-lane sums
// do not (a unit's sub-units sit in adjacent lanes of one pass and are
// combined in a fixed order), so any count whose chunk holds a one-group row
// gives the bits of the class's own kernel.  Fewer sub-units hold fewer
// registers, and the fused kernel holds the registers of its largest body.
__host__ __device__ constexpr int fuse_ss(int bits, int M, int slices) {
  return chunk_slices(bits, M, 1) >= slices ? 1 : chunk_slices(bits, M, 2) >= slices ? 2 : kStageSubMax;
}
// Slices per staged chunk of a streamed row in the fused launch, and slices
// per load group of its body.  The fused kernel holds the registers of its
// largest body, and the streamed body is the largest, so these choices set
// the resident waves of the whole launch.  Measured on the Llama-3-8B decode
// step (M = 1): INT4 down rows (7 slices) run fastest in chunks of 2 with
// one staging sub-unit; INT2 down rows (4 slices) in chunks of 1 (one
// sub-unit: 77 registers, 6 waves per SIMD, against 140 and 3 waves for one
// chunk of 4, which saves the restaging but starves the rest of the launch:
// INT2 step 12.6 -> 11.1 us).  Loads of one slice per group (a wave streams
// its rows slice by slice) hold the fewest registers again (INT4 step
// 15.5 -> 15.3 us).
__host__ __device__ constexpr int fuse_stream_chunk(int bits) { return bits == 2 ? 1 : 2; }
constexpr int kFuseStreamNL = 1;

// Every one-workgroup-per-tile class of one width in one launch.  Between
// two launches on a stream the first one's last workgroups finish before
// the second one's first start; in one grid the dispatcher starts the next
// class's workgroups as soon as CUs free up, so the launch pays one ramp and
// one tail instead of one per class.  The classes are ordered longest tiles
// first, so the workgroups dispatched last are the shortest.  Each
// workgroup runs the body of its class's load-group configuration (a branch
// uniform over the workgroup), with the staging of fuse_ss; the LDS is the
// largest class's.  BODIES is the set of load-group configurations the
// launch's classes use (bit 0: rows of one slice, bit 1: rows of two
// slices, bit 2: streamed rows): a kernel holds the registers of the largest
// body it contains, so it contains only those.
template <int ACT, int M, int BITS, int BODIES>
__global__ __launch_bounds__(kThreads) void gemv_group_fused_kernel(const uint8_t *__restrict__ plan,
                                                                    FuseArgs fa) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int b = blockIdx.x;
  int cls = fa.cls[0], one = fa.one[0], s0 = 0, s1 = fa.start[1];
#pragma unroll
  for (int j = 1; j < kFuseMax; ++j)
    if (j < fa.n && b >= fa.start[j]) {
      cls = fa.cls[j];
      one = fa.one[j];
      s0 = fa.start[j];
      s1 = fa.start[j + 1];
    }
  const int G = s1 - s0, w = b - s0;
  if constexpr ((BODIES & 1) != 0)
    if (one == 1) {
      group_body<ACT, M, BITS, fuse_ss(BITS, M, 1), 1, true, false>(plan, cls, 1, G, w, lds);
      return;
    }
  if constexpr ((BODIES & 2) != 0)
    if (one == 2) {
      group_body<ACT, M, BITS, fuse_ss(BITS, M, 2), 2, true, false>(plan, cls, 1, G, w, lds);
      return;
    }
  if constexpr ((BODIES & 4) != 0)
    if (one == 0)
      group_body<ACT, M, BITS, fuse_ss(BITS, M, fuse_stream_chunk(BITS)), kFuseStreamNL, false, false>(plan, cls, 1, G, w, lds);
}

typedef void (*GroupKernel)(const uint8_t *, int, int);

// one: 0 streamed rows, 1 rows of one slice (one-slice load groups), 2 rows
// of two slices; pipe: the software-pipelined persistent body
template <int ACT, int M, int BITS, int SS>
GroupKernel group_kernel_ss(int one, bool pipe) {
  if (one == 1)
    return pipe ? gemv_group_kernel<ACT, M, BITS, SS, 1, true, true> : gemv_group_kernel<ACT, M, BITS, SS, 1, true, false>;
  if (one == 2)
    return pipe ? gemv_group_kernel<ACT, M, BITS, SS, 2, true, true> : gemv_group_kernel<ACT, M, BITS, SS, 2, true, false>;
  return gemv_group_kernel<ACT, M, BITS, SS, kGroupNL, false, false>;
}

template <int ACT, int M, int BITS>
GroupKernel group_kernel_bits(int ss, int one, bool pipe) {
  if (chunk_slices(BITS, M, ss) < 1) return nullptr;   // not a configuration the plan picks
  if (ss == 1) return group_kernel_ss<ACT, M, BITS, 1>(one, pipe);
  if (ss == 2) return group_kernel_ss<ACT, M, BITS, 2>(one, pipe);
  return group_kernel_ss<ACT, M, BITS, 4>(one, pipe);
}

template <int ACT, int M>
GroupKernel group_kernel_m(int bits, int ss, int one, bool pipe) {
  if (bits == 8) return group_kernel_bits<ACT, M, 8>(ss, one, pipe);
  return bits == 4 ? group_kernel_bits<ACT, M, 4>(ss, one, pipe) : group_kernel_bits<ACT, M, 2>(ss, one, pipe);
}

GroupKernel group_kernel(int act, int M, int bits, int ss, int one, bool pipe) {
  const bool bf = act == GQ_BF16;
  switch (M) {
    case 1: return bf ? group_kernel_m<0, 1>(bits, ss, one, pipe) : group_kernel_m<1, 1>(bits, ss, one, pipe);
    case 2: return bf ? group_kernel_m<0, 2>(bits, ss, one, pipe) : group_kernel_m<1, 2>(bits, ss, one, pipe);
    case 3: return bf ? group_kernel_m<0, 3>(bits, ss, one, pipe) : group_kernel_m<1, 3>(bits, ss, one, pipe);
    default: return bf ? group_kernel_m<0, 4>(bits, ss, one, pipe) : group_kernel_m<1, 4>(bits, ss, one, pipe);
  }
}

typedef void (*FusedKernel)(const uint8_t *, FuseArgs);

template <int ACT, int M, int BITS>
FusedKernel fused_kernel_b(int bodies) {
  switch (bodies) {
    case 1: return gemv_group_fused_kernel<ACT, M, BITS, 1>;
    case 2: return gemv_group_fused_kernel<ACT, M, BITS, 2>;
    case 3: return gemv_group_fused_kernel<ACT, M, BITS, 3>;
    case 4: return gemv_group_fused_kernel<ACT, M, BITS, 4>;
    case 5: return gemv_group_fused_kernel<ACT, M, BITS, 5>;
    case 6: return gemv_group_fused_kernel<ACT, M, BITS, 6>;
    default: return gemv_group_fused_kernel<ACT, M, BITS, 7>;
  }
}

template <int ACT, int M>
FusedKernel fused_kernel_m(int bits, int bodies) {
  if (bits == 8) return fused_kernel_b<ACT, M, 8>(bodies);
  return bits == 4 ? fused_kernel_b<ACT, M, 4>(bodies) : fused_kernel_b<ACT, M, 2>(bodies);
}

// bodies: the set of load-group configurations of the launch's classes
// (bit 0: one slice, bit 1: two slices, bit 2: streamed)
FusedKernel fused_kernel(int act, int M, int bits, int bodies) {
  const bool bf = act == GQ_BF16;
  switch (M) {
    case 1: return bf ? fused_kernel_m<0, 1>(bits, bodies) : fused_kernel_m<1, 1>(bits, bodies);
    case 2: return bf ? fused_kernel_m<0, 2>(bits, bodies) : fused_kernel_m<1, 2>(bits, bodies);
    case 3: return bf ? fused_kernel_m<0, 3>(bits, bodies) : fused_kernel_m<1, 3>(bits, bodies);
    default: return bf ? fused_kernel_m<0, 4>(bits, bodies) : fused_kernel_m<1, 4>(bits, bodies);
  }
}

// Resident workgroups per CU of a kernel at an LDS size, and CUs of the
// current device; each queried once and kept.
int resident_grid(GroupKernel k, int lds) {
  struct Entry { GroupKernel k; int lds; int dev; int grid; };
  static std::mutex mu;
  static Entry cache[256];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].k == k && cache[i].lds == lds && cache[i].dev == dev) return cache[i].grid;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(k), kThreads,
                                                   lds) != hipSuccess)
    return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int grid = per_cu * cus;
  if (used < 256) cache[used++] = {k, lds, dev, grid};
  return grid;
}

// Kernel configuration of one bit-width of a linear: the single-linear
// launch's choices (staging sub-units, one load group per row or streamed
// rows), with R and NL fixed for the group.
struct WidthCfg {
  int ss, one, lds;
};

WidthCfg width_cfg(int bits, int K, int M) {
  const int ns = (K * bits / 8 + 1023) / 1024;
  const int units = M * kLanes * (8 / bits) * ns;
  const int need = (units + kThreads - 1) / kThreads;
  WidthCfg c;
  c.ss = need <= 1 ? 1 : (need <= 2 ? 2 : kStageSubMax);
  // one-load-group rows: 1 or 2 slices (the load group's size), else 0
  c.one = (ns <= kGroupNL && ns <= chunk_slices(bits, M, c.ss)) ? ns : 0;
  c.lds = stage_bytes(bits, M, ns, c.ss);
  return c;
}

// key of a kernel class: width (4, 2, 8 -> 0, 16, 32), then staging and
// load-group configuration
inline int class_key(int bits, const WidthCfg &c) { return (bits == 4 ? 0 : bits == 2 ? 16 : 32) + c.ss * 3 + c.one; }
inline int key_bits(int key) { return key < 16 ? 4 : key < 32 ? 2 : 8; }

}  // namespace

gq_status gemv_group_plan(int count, const gq_group_item *items, int M, gq_dtype act, void *plan,
                          size_t plan_bytes, size_t *need) {
  if (!items) return GQ_ERR_NULL_ARG;
  if (count < 1 || count > 65535 || M < 1 || M > kGemvMaxM) return GQ_ERR_SHAPE;
  if (act != GQ_BF16 && act != GQ_FP16) return GQ_ERR_DTYPE;
  // pass 1: check every item, count segments and classes
  int nkeys = 0, keys[kGroupMaxClasses];
  int64_t nseg = 0;
  for (int i = 0; i < count; ++i) {
    const gq_group_item &it = items[i];
    LayoutDev L;
    gq_status st = make_layout(&it.layout, &L);
    if (st != GQ_OK) return st;
    if (L.N == 0) continue;
    if ((st = check_ptr16(it.x)) != GQ_OK) return st;
    if ((st = check_ptr16(it.codes)) != GQ_OK) return st;
    if (!it.scales || !it.zeros || !it.y) return GQ_ERR_NULL_ARG;
    if (((uintptr_t)it.scales & 1u) || ((uintptr_t)it.y & 1u)) return GQ_ERR_ALIGNMENT;
    int prev = -1;
    for (int b = 0; b < L.nblocks; ++b) {
      const int bits = block_info(L, b).bits;
      if (bits != prev) ++nseg;
      prev = bits;
      const int key = class_key(bits, width_cfg(bits, L.K, M));
      bool seen = false;
      for (int k = 0; k < nkeys; ++k) seen |= keys[k] == key;
      if (!seen) keys[nkeys++] = key;   // at most 3 widths x 3 x 3 = 27 keys
    }
  }
  if (nseg > INT32_MAX / 2) return GQ_ERR_SHAPE;
  const size_t items_off = (sizeof(GroupPlanHeader) + 15) & ~(size_t)15;
  const size_t segs_off = items_off + (size_t)count * sizeof(GroupItemDev);
  const size_t bytes = segs_off + (size_t)nseg * sizeof(GroupSeg);
  if (need) *need = bytes;
  if (!plan) return GQ_OK;
  if (plan_bytes < bytes) return GQ_ERR_WORKSPACE;
  uint8_t *P = static_cast<uint8_t *>(plan);
  memset(P, 0, bytes);
  GroupPlanHeader &H = *reinterpret_cast<GroupPlanHeader *>(P);
  H.magic = kGroupMagic;
  H.version = kGroupVersion;
  H.bytes = bytes;
  H.count = count;
  H.M = M;
  H.act = act;
  H.items_off = items_off;
  H.segs_off = segs_off;
  GroupItemDev *dst = reinterpret_cast<GroupItemDev *>(P + items_off);
  for (int i = 0; i < count; ++i) {
    GroupItemDev &D = dst[i];
    make_layout(&items[i].layout, &D.L);
    D.x = items[i].x;
    D.codes = items[i].codes;
    D.scales = items[i].scales;
    D.zeros = items[i].zeros;
    D.y = items[i].y;
    D.uniform = D.L.nblocks == 1;
  }
  // classes in key order; inside a class, linears in call order and their
  // runs of same-width blocks in block order
  for (int a = 1; a < nkeys; ++a)
    for (int b = a; b > 0 && keys[b - 1] > keys[b]; --b) {
      const int tk = keys[b]; keys[b] = keys[b - 1]; keys[b - 1] = tk;
    }
  GroupSeg *segs = reinterpret_cast<GroupSeg *>(P + segs_off);
  int si = 0;
  for (int k = 0; k < nkeys; ++k) {
    GroupClass &C = H.cls[k];
    C.seg0 = si;
    C.bits = key_bits(keys[k]);
    C.ss = (keys[k] & 15) / 3;
    C.one = (keys[k] & 15) % 3;
    int tiles = 0;
    int64_t cbytes = 0;
    for (int i = 0; i < count; ++i) {
      const LayoutDev &L = dst[i].L;
      if (L.N == 0) continue;
      const WidthCfg c = width_cfg(C.bits, L.K, M);
      if (class_key(C.bits, c) != keys[k]) continue;
      for (int b = 0; b < L.nblocks;) {
        if (block_info(L, b).bits != C.bits) { ++b; continue; }
        int e = b;
        while (e < L.nblocks && block_info(L, e).bits == C.bits) ++e;
        const int tile = group_tile(C.bits, M);
        const int t0 = b * L.block_n / tile;
        const int t1 = e == L.nblocks ? (L.N + tile - 1) / tile : e * L.block_n / tile;
        const BlockInfo bi = block_info(L, b);
        const int64_t rb = (int64_t)L.K * C.bits / 8;
        GroupSeg &S = segs[si++];
        S.codes = reinterpret_cast<const uint8_t *>(items[i].codes) + bi.code_off;
        S.scales = static_cast<const uint16_t *>(items[i].scales) + bi.grp_off;
        S.zeros = static_cast<const uint8_t *>(items[i].zeros) + bi.grp_off;
        S.item = i;
        S.tile0 = t0;
        S.ntiles = t1 - t0;
        S.ctile0 = tiles;
        S.rows = (e == L.nblocks ? L.N : e * L.block_n) - b * L.block_n;
        S.tile_bytes = (int32_t)(rb * tile);
        S.cbyte0 = cbytes;
        tiles += S.ntiles;
        cbytes += (int64_t)S.ntiles * S.tile_bytes;
        b = e;
      }
      if (c.lds > C.lds) C.lds = c.lds;
    }
    C.nseg = si - C.seg0;
    C.tiles = tiles;
    C.bytes = cbytes;
  }
  H.nclass = nkeys;
  H.nseg = si;
  return GQ_OK;
}

gq_status gemv_group_check(const void *plan) {
  if (!plan) return GQ_ERR_NULL_ARG;
  const GroupPlanHeader &H = *static_cast<const GroupPlanHeader *>(plan);
  if (H.magic != kGroupMagic || H.version != kGroupVersion) return GQ_ERR_SHAPE;
  if (H.count < 1 || H.M < 1 || H.M > kGemvMaxM || (H.act != GQ_BF16 && H.act != GQ_FP16))
    return GQ_ERR_SHAPE;
  if (H.nclass < 0 || H.nclass > kGroupMaxClasses || H.nseg < 0) return GQ_ERR_SHAPE;
  if (H.items_off + (uint64_t)H.count * sizeof(GroupItemDev) > H.segs_off ||
      H.segs_off + (uint64_t)H.nseg * sizeof(GroupSeg) != H.bytes)
    return GQ_ERR_SHAPE;
  int seg = 0;
  for (int c = 0; c < H.nclass; ++c) {
    const GroupClass &C = H.cls[c];
    if (C.seg0 != seg || C.nseg < 1 || (C.bits != 4 && C.bits != 2 && C.bits != 8) ||
        (C.ss != 1 && C.ss != 2 && C.ss != 4) || C.one < 0 || C.one > kGroupNL || C.lds < 0 ||
        C.lds > kLdsBytes || C.tiles < 1 || C.bytes < C.tiles)
      return GQ_ERR_SHAPE;
    seg += C.nseg;
  }
  return seg == H.nseg ? GQ_OK : GQ_ERR_SHAPE;
}

hipError_t launch_gemv_group(const GroupPlanHeader &H, const void *plan_dev, hipStream_t s) {
  const uint8_t *p = static_cast<const uint8_t *>(plan_dev);
  FuseArgs fuse[3] = {};                     // one-workgroup-per-tile classes of INT4, INT2, 8-bit
  int fuse_lds[3] = {0, 0, 0};
  for (int c = 0; c < H.nclass; ++c) {
    const GroupClass &C = H.cls[c];
    // a class with many tiles per resident workgroup runs as a persistent
    // grid (software pipelined over a byte-balanced contiguous tile range
    // when its rows fit one load group, else taking chunks of kGroupChunk
    // tiles in turn); a small one as one workgroup per tile (the hardware
    // dispatcher then overlaps the workgroups' start and end, and no
    // workgroup pays the pipeline's extra registers for a single tile)
    const GroupKernel kp = group_kernel(H.act, H.M, C.bits, C.ss, C.one, true);
    if (!kp) return hipErrorInvalidConfiguration;
    const int resident = resident_grid(kp, C.lds);
    if (resident <= 0) return hipErrorInvalidConfiguration;
    if ((int64_t)C.tiles >= (int64_t)kGroupPersistTiles * resident) {
      const int grid = resident < C.tiles ? resident : C.tiles;
      hipLaunchKernelGGL(kp, dim3(grid), dim3(kThreads), C.lds, s, p, c, kGroupChunk);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      continue;
    }
    const int wi = C.bits == 4 ? 0 : C.bits == 2 ? 1 : 2;
    FuseArgs &F = fuse[wi];
    if (F.n >= kFuseMax) return hipErrorInvalidConfiguration;
    F.cls[F.n] = c;
    F.one[F.n] = C.one;
    ++F.n;
    // a streamed class stages chunks of fuse_ss's size in the fused launch
    const int lds = C.one ? C.lds : stage_bytes(C.bits, H.M, 1 << 20, fuse_ss(C.bits, H.M, fuse_stream_chunk(C.bits)));
    if (lds > fuse_lds[wi]) fuse_lds[wi] = lds;
  }
  for (int wi = 0; wi < 3; ++wi) {
    FuseArgs &F = fuse[wi];
    if (F.n == 0) continue;
    if (F.n == 1) {                          // a class alone keeps its own kernel's registers
      const GroupClass &C = H.cls[F.cls[0]];
      const GroupKernel k = group_kernel(H.act, H.M, C.bits, C.ss, C.one, false);
      if (!k) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(k, dim3(C.tiles), dim3(kThreads), C.lds, s, p, F.cls[0], 1);
    } else {
      // longest tiles first: bytes per tile, C.bytes / C.tiles, decreasing
      for (int a = 1; a < F.n; ++a)
        for (int b = a; b > 0; --b) {
          const GroupClass &P = H.cls[F.cls[b - 1]], &Q = H.cls[F.cls[b]];
          if (P.bytes * Q.tiles >= Q.bytes * P.tiles) break;
          const int tc = F.cls[b], to = F.one[b];
          F.cls[b] = F.cls[b - 1];
          F.one[b] = F.one[b - 1];
          F.cls[b - 1] = tc;
          F.one[b - 1] = to;
        }
      int64_t grid = 0;
      for (int j = 0; j < F.n; ++j) {
        F.start[j] = (int32_t)grid;
        grid += H.cls[F.cls[j]].tiles;
      }
      if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
      F.start[F.n] = (int32_t)grid;
      int bodies = 0;
      for (int j = 0; j < F.n; ++j) bodies |= F.one[j] == 1 ? 1 : F.one[j] == 2 ? 2 : 4;
      const FusedKernel k = fused_kernel(H.act, H.M, wi == 0 ? 4 : wi == 1 ? 2 : 8, bodies);
      hipLaunchKernelGGL(k, dim3((uint32_t)grid), dim3(kThreads), fuse_lds[wi], s, p, F);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gq
