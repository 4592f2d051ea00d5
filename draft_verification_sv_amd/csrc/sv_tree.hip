// sv_tree.hip -- tree verification: multi-round speculative sampling over the
// candidates of each node of a draft tree.
//
// The pages name tree drafters (wispaper Q&A on block-diffusion decode
// failures, section "Why is a fixed block size a failure mode in
// production?": Bastion's budget-aware draft trees; its source list: D2SD's
// confidence-guided prefix trees) but give no rule for verifying several
// candidates.  The rule here is multi-round speculative sampling (Miao et al.,
// SpecInfer, ASPLOS 2024): the children of a node were drawn independently
// from the drafter's distribution q of that position (a block drafter's
// position-wise marginal: dense draft row depth(u) of the request) and are
// tested in turn against the current target r, starting from r = p (the
// node's target row); a rejection replaces r by norm(max(0, r - q)); when
// every child fails the token is drawn from that residual, and at a leaf a
// bonus token from p.  Rejection correction keeps the target distribution
// ("Pith review of DBLAST", "Assumptions & free parameters").
//
// After k rejections at a node the target is max(0, p - c_k q) / Z_k with
// c_1 = 1, c_{k+1} = c_k + Z_k and Z_k = sum_v max(0, p_v - c_k q_v): one
// scalar per rejection instead of a vector (a residual emptied by rounding
// resets the target to p, as the block rule does: c_k = 0, Z_k = 1).  The c_k
// do not depend on the walk's random tests, so the masses Z_k of every node
// are formed beforehand, one launch per k, over blocks of (node, chunk of the
// rows); one wave per request then walks the tree, and the token is drawn by
// the block draw's sums and pick with the draft row scaled by c (its
// log-normaliser lowered by ln c).
//
// Launches: k_tree_prep (a block per request: depths, child counts, checks),
// k_tree_mass for k = 1 .. max_kids - 1, k_tree_walk (a wave per request), and
// the record draw (sums, pick) of sv_sample.hip.
#include <math.h>

#include "sv_device.hpp"
#include "sv_draw.hpp"
#include "sv_host.hpp"

namespace sv {

constexpr int kTreeNT = 256;
constexpr int kTreeMaxKids = 16;    // children tested per node
constexpr int kTreeMaxNodes = 1024; // nodes of one request (staged in LDS by the walk)
constexpr int kTreeChunk = 4096;    // values of a row per mass block (the draw's chunk)
constexpr int kTreeMaxReq = 1024;   // requests of one call (the mass kernel scans their counts in LDS)
constexpr int kTreeMassGrid = 1024; // mass blocks: four 256-thread blocks per compute unit

struct TreeNode {
  int32_t depth, kids, req, valid;
};

struct TreeArgs {
  const void* tgt;
  int dtype;
  int64_t tgt_ld;
  int V;
  const int32_t* node_off;
  const int32_t* parent;
  const int32_t* token;
  int R, b, max_nodes, max_kids, S;
  const float* T;
  const int32_t* row_argmax;
  const float* row_cut;
  const double* row_kept;
  const void* draft;
  int ddtype;
  int64_t draft_ld;
  const int32_t* dargmax;
  const double* dlse;
  const uint64_t* seed;
  int32_t* n_acc;
  int32_t* path;
  int32_t* stop_node;
  double* p_out;
  double* q_out;
  float* u_out;
  TreeNode* nodes;  // [max_nodes]
  double* zpart;    // [max_nodes][max_kids - 1][S]: partial masses Z_k per chunk
  int2* order;      // [max_nodes]: request r's nodes with >= 2 children, by child count descending,
                    // at node_off[r] ...: {local index, depth}
  int32_t* khist;   // [R][kTreeMaxKids + 1]: request r's count of such nodes per child count
  DrawRec* rec;     // [R]
  uint32_t* status;
};

// Z_m of a node from its pass-m chunk partials zp[0 .. S-1], summed in chunk
// order (the mass passes and the walk form it alike, bit for bit); loads in
// batches of 16, all of a batch in flight before any is added.
__device__ __forceinline__ double zsum(const double* zp, int S) {
  double z = 0.0;
  for (int s0 = 0; s0 < S; s0 += 16) {
    double v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = s0 + k < S ? zp[s0 + k] : 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (s0 + k < S) z += v[k];
  }
  return z;
}

// Whether request r's node range is usable: n0 >= 0, 1 <= N <= kTreeMaxNodes,
// inside the node count node_off[R] and the capacity max_nodes.
__device__ __forceinline__ bool tree_range_ok(const TreeArgs& a, int r, int& n0, int& N) {
  n0 = a.node_off[r];
  N = a.node_off[r + 1] - n0;
  const long long end = static_cast<long long>(n0) + N;
  return n0 >= 0 && N >= 1 && N <= kTreeMaxNodes && end <= a.max_nodes && end <= a.node_off[a.R];
}

// Whether a node record is usable by request r: written by r's checks, with
// depth and child count in range (a node with children lies above depth b).
// Records of requests whose offsets overlap (malformed node_off) or left from
// an earlier call fail it, so no index below is taken from unchecked data.
__device__ __forceinline__ bool tree_node_ok(const TreeArgs& a, const TreeNode& nd, int r) {
  return nd.valid == 1 && nd.req == r && nd.depth >= 0 && nd.depth <= a.b && nd.kids >= 0 &&
         nd.kids <= a.max_kids && (nd.kids == 0 || nd.depth < a.b);
}

// Depths (by climbing the parents: at most b + 1 steps) and child counts of
// request r's nodes, and the checks: the root's parent is -1, every other
// parent precedes its child, depth <= b, at most max_kids children.
__global__ __launch_bounds__(kTreeNT) void k_tree_prep(TreeArgs a) {
  __shared__ int kids[kTreeMaxNodes];
  __shared__ int depth[kTreeMaxNodes];
  __shared__ int hist[kTreeMaxKids + 1], cursor[kTreeMaxKids + 1];
  __shared__ int bad;
  const int r = blockIdx.x, tid = threadIdx.x;
  int n0, N;
  const bool range = tree_range_ok(a, r, n0, N);
  if (tid <= kTreeMaxKids) a.khist[r * (kTreeMaxKids + 1) + tid] = 0;  // rewritten below for a usable request
  if (!range) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_TREE);
    return;
  }
  if (tid == 0) bad = 0;
  for (int j = tid; j < N; j += kTreeNT) kids[j] = 0;
  __syncthreads();
  const int32_t* par = a.parent + n0;
  for (int j = tid; j < N; j += kTreeNT) {
    const int pj = par[j];
    if (j == 0 ? pj != -1 : (pj < 0 || pj >= j)) {
      bad = 1;
      continue;
    }
    if (j > 0) atomicAdd(&kids[pj], 1);
  }
  __syncthreads();
  if (bad) {  // climbing a malformed tree could loop; every node is marked unusable
    for (int j = tid; j < N; j += kTreeNT) a.nodes[n0 + j] = TreeNode{0, 0, r, 0};
    if (tid == 0) raise_status(a.status, SV_ST_BAD_TREE);
    return;
  }
  for (int j = tid; j < N; j += kTreeNT) {
    int d = 0, u = j;
    while (u > 0 && d <= a.b) {  // parents precede children, so this ends
      u = par[u];
      ++d;
    }
    if (d > a.b || kids[j] > a.max_kids) bad = 1;
    a.nodes[n0 + j] = TreeNode{d, kids[j], r, 1};
    depth[j] = d;
  }
  if (tid <= kTreeMaxKids) {
    hist[tid] = 0;
    cursor[tid] = 0;
  }
  __syncthreads();
  if (bad) {
    for (int j = tid; j < N; j += kTreeNT) a.nodes[n0 + j].valid = 0;
    if (tid == 0) raise_status(a.status, SV_ST_BAD_TREE);
  }
  // the nodes the mass passes take (>= 2 children; none for a greedy or
  // malformed request), grouped by child count, most children first: pass k
  // takes the first sum_{v > k} hist[v] of them
  const bool masses = !bad && a.T[r] > 0.0f;
  if (masses)
    for (int j = tid; j < N; j += kTreeNT)
      if (kids[j] >= 2) atomicAdd(&hist[kids[j]], 1);
  __syncthreads();
  if (tid <= kTreeMaxKids) a.khist[r * (kTreeMaxKids + 1) + tid] = masses && tid >= 2 ? hist[tid] : 0;
  if (masses)
    for (int j = tid; j < N; j += kTreeNT) {
      const int v = kids[j];
      if (v < 2) continue;
      int start = 0;
      for (int u = v + 1; u <= kTreeMaxKids; ++u) start += hist[u];
      a.order[n0 + start + atomicAdd(&cursor[v], 1)] = make_int2(j, depth[j]);
    }
}

// Pass k: for every node with more than k children, the partial masses over
// each chunk of 4096 values of sum_v max(0, p_v - c_k q_v) (p: the node's
// target row with its cut; q: the draft row of the node's depth).  Greedy
// requests (T = 0) need no masses.  A fixed grid walks the pass's (node,
// chunk) items: each block scans the requests' counts of nodes with more than
// k children (from the prep's per-count histograms) and takes items
// blockIdx.x, blockIdx.x + gridDim.x, ...; so no block is launched for a node
// without work.  Per block, up to kMassBatch of its items are set up at once
// (one item per thread: node, rows, cut, normalisers, c_k into LDS), then
// walked in order with the next item's four 16-byte loads per thread issued
// before the current item is computed.  Only values with p > c q carry mass:
// ln p = l / T - kept against ln(c q) = d / T - (lse - ln c), two FMAs in
// double; their (l, d) pairs are packed into the wave's list, and the double
// exponentials run over the list with every lane busy.
constexpr int kMassBatch = 64;  // items set up at once per block (LDS for four blocks per CU)

struct MassItem {
  const char* tp;  // target row
  const char* dp;  // draft row
  double kept, dl, invT;
  float cut;
  int zslot;       // index of this item's partial in zpart
};

template <int DT, int DDT>
__global__ __launch_bounds__(kTreeNT) void k_tree_mass(TreeArgs a, int k) {
  __shared__ double etab[kExpTab];
  __shared__ double red[kTreeNT / kWave];
  __shared__ int scan[kTreeMaxReq + 1];  // exclusive scan of the requests' active node counts
  __shared__ int wtot[kTreeNT / kWave];
  __shared__ MassItem items[kMassBatch];
  __shared__ float2 list[kTreeNT * 16];  // per wave: the (l, d) pairs of its values with p > c q
  const int tid = threadIdx.x, lane = tid & (kWave - 1), R = a.R;
  exp_table_init(etab);
  // requests' counts in contiguous runs per thread, then a block scan
  const int per = (R + kTreeNT - 1) / kTreeNT;
  const int r0 = min(R, tid * per), r1 = min(R, r0 + per);
  int mine = 0;
  for (int r = r0; r < r1; ++r) {
    const int32_t* h = a.khist + r * (kTreeMaxKids + 1);
    int c = 0;
    for (int v = k + 1; v <= kTreeMaxKids; ++v) c += h[v];
    scan[r] = c;  // the count, turned into its exclusive prefix below
    mine += c;
  }
  int total;
  int run = block_excl_scan_i32<kTreeNT>(mine, wtot, &total);
  for (int r = r0; r < r1; ++r) {
    const int c = scan[r];
    scan[r] = run;
    run += c;
  }
  if (tid == 0) scan[R] = total;
  __syncthreads();  // scan and table
  const int S = a.S, V = a.V, NG = groups_of(V);
  const long long n_items = static_cast<long long>(total) * S;
  const long long mine_items = n_items > blockIdx.x ? (n_items - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  for (long long j0 = 0; j0 < mine_items; j0 += kMassBatch) {
    const int nj = static_cast<int>(min<long long>(kMassBatch, mine_items - j0));
    // set-up of items j0 .. j0 + nj - 1, one per thread
    if (tid < nj) {
      const long long it = blockIdx.x + (j0 + tid) * gridDim.x;
      const int pos = static_cast<int>(it / S), ch = static_cast<int>(it % S);
      int lo = 0, hi = R;  // the request r with scan[r] <= pos < scan[r + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (scan[mid] <= pos) lo = mid;
        else hi = mid;
      }
      const int r = lo;
      const int n0 = a.node_off[r];
      const int2 e = a.order[n0 + (pos - scan[r])];
      const int g = n0 + e.x;
      const int64_t drow = static_cast<int64_t>(r) * a.b + min(max(e.y, 0), a.b - 1);
      const float T = a.T[r];
      const float cut = a.row_cut[g];
      const double kept = a.row_kept[g];
      const double dlse = a.dlse[drow];
      // c_k: c_1 = 1, c_{m+1} = c_m + Z_m (a mass emptied by rounding resets the target to p: c = 0, Z = 1)
      const size_t zbase = static_cast<size_t>(g) * (a.max_kids - 1) * S;
      double c = 1.0;
      for (int m = 1; m < k; ++m) {
        const double Z = zsum(a.zpart + zbase + static_cast<size_t>(m - 1) * S, S);
        c = Z > 0.0 ? c + Z : 1.0;
      }
      MassItem I;
      I.tp = row_ptr(a.tgt, DT, g, a.tgt_ld);
      I.dp = row_ptr(a.draft, DDT, drow, a.draft_ld);
      I.kept = kept;
      I.dl = dlse - log(c);  // c q = exp(d / T - (lse - ln c))
      I.invT = 1.0 / static_cast<double>(T);
      I.cut = cut;
      I.zslot = static_cast<int>(zbase + static_cast<size_t>(k - 1) * S + ch);
      items[tid] = I;
    }
    __syncthreads();
    // this thread's two 8-value groups of item j's chunk
    auto gabs = [&](int j, int cg) {
      const long long it = blockIdx.x + (j0 + j) * gridDim.x;
      return static_cast<int>(it % S) * (kTreeChunk / 8) + cg;
    };
    const int c0 = tid, c1 = tid + kTreeNT;
    uint4 t00, t01, t10, t11, d00, d01, d10, d11;
    auto issue = [&](int j) {
      const MassItem& I = items[j];
      const int ga = min(gabs(j, c0), NG - 1), gb = min(gabs(j, c1), NG - 1);  // clamped in-bounds (unused there)
      raw8<DT>(I.tp, ga, V, t00, t01);
      raw8<DT>(I.tp, gb, V, t10, t11);
      raw8<DDT>(I.dp, ga, V, d00, d01);
      raw8<DDT>(I.dp, gb, V, d10, d11);
    };
    issue(0);
    for (int j = 0; j < nj; ++j) {
      const MassItem I = items[j];
      const int ga = gabs(j, c0), gb = gabs(j, c1);
      float l[16], d[16];
      decode8<DT>(t00, t01, ga, V, ga < NG, l);
      decode8<DT>(t10, t11, gb, V, gb < NG, l + 8);
      decode8<DDT>(d00, d01, ga, V, ga < NG, d);
      decode8<DDT>(d10, d11, gb, V, gb < NG, d + 8);
      if (j + 1 < nj) issue(j + 1);  // the next item's loads, in flight while this one is formed
      int cnt = 0;
      bool keep[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        keep[q] = l[q] > -INFINITY && l[q] >= I.cut &&
                  fma(static_cast<double>(l[q]), I.invT, -I.kept) > fma(static_cast<double>(d[q]), I.invT, -I.dl);
        cnt += keep[q] ? 1 : 0;
      }
      const int inc = wave_incl_scan_i32(cnt);
      const int n_list = bcast_i32(inc, kWave - 1);
      float2* wl = list + (tid / kWave) * (kWave * 16);
      int o = inc - cnt;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (keep[q]) wl[o++] = make_float2(l[q], d[q]);
      __syncwarp();
      double part = 0.0;
      for (int e = lane; e < n_list; e += kWave) {
        const float2 v = wl[e];
        const double w = exp_tab(fma(static_cast<double>(v.x), I.invT, -I.kept), etab) -
                         exp_tab(fma(static_cast<double>(v.y), I.invT, -I.dl), etab);
        part += w > 0.0 ? w : 0.0;
      }
      const double tot = block_sum_f64<kTreeNT>(part, red);  // its leading barrier also ends the list's reads
      if (tid == 0) a.zpart[I.zslot] = tot;
    }
    __syncthreads();  // items[] is rewritten by the next set-up
  }
}

// The walk, one wave per request: from the root, each node's children in
// index order are tested against the current target; an acceptance moves to
// the child, and the walk ends at a leaf (bonus draw from its p) or when every
// child fails (residual draw).  The test of node j takes Philox word 0 at
// counter (j - 1, r, 0, 0); the draw record's n is the stopping node, whose
// word 1 the pick takes.
// Everything a test reads is staged in LDS first, in two load rounds over the
// request's nodes (lanes over nodes): parents, tokens, node records, cuts,
// normalisers and argmaxes, the drafter's per-depth statistics; then, per
// node, p of its token in its parent's target row (with the cut), q in the
// draft row of the parent's depth, and its uniform -- none of which depends
// on the walk.  The walk itself rescales p by the current residual (c, Z)
// and reads LDS only, apart from the masses Z_m of a node at which m
// children have been rejected (summed in chunk order, as the mass passes
// form c_k).
template <int DT, int DDT>
__global__ __launch_bounds__(kWave) void k_tree_walk(TreeArgs a) {
  __shared__ int par[kTreeMaxNodes], tok[kTreeMaxNodes], am[kTreeMaxNodes];
  __shared__ int2 kd[kTreeMaxNodes];      // {kids, depth}; kids = -1: the record fails its checks
  __shared__ float cutv[kTreeMaxNodes];
  __shared__ double keptv[kTreeMaxNodes];
  __shared__ double2 pq[kTreeMaxNodes];   // node j's token: p in its parent's target row (with the cut), q in the draft row
  __shared__ float uv[kTreeMaxNodes];     // node j's uniform (word 0 of Philox at counter (j - 1, r, 0, 0))
  __shared__ double dlse_d[64];           // the drafter's statistics per depth (b <= 64)
  __shared__ int dam_d[64];
  __shared__ double etab[kExpTab];
  const int r = blockIdx.x, lane = threadIdx.x;
  int n0, N;
  DrawRec& rec = a.rec[r];
  exp_table_init(etab);
  const bool range = tree_range_ok(a, r, n0, N);
  const bool ok = range && a.nodes[n0].valid;
  auto fail = [&](bool bad_tree) {
    if (lane == 0) {
      if (bad_tree) raise_status(a.status, SV_ST_BAD_TREE);
      a.n_acc[r] = 0;
      a.stop_node[r] = 0;
      rec.mode = kDrawNone;
    }
  };
  if (!ok) {
    fail(false);  // reported by the checks
    return;
  }
  const float T = a.T[r];
  const bool greedy = T == 0.0f;
  const double invT = 1.0 / static_cast<double>(T);
  const uint64_t seed = *a.seed;
  const int V = a.V, b = a.b;
  // first loads: per node and per depth
  for (int j = lane; j < N; j += kWave) {
    const int g = n0 + j;
    const TreeNode nd = a.nodes[g];
    par[j] = a.parent[g];
    tok[j] = a.token[g];
    am[j] = a.row_argmax[g];
    cutv[j] = a.row_cut[g];
    keptv[j] = a.row_kept[g];
    kd[j] = tree_node_ok(a, nd, r) ? make_int2(nd.kids, nd.depth) : make_int2(-1, 0);
  }
  if (lane < b) {
    dlse_d[lane] = greedy ? 0.0 : a.dlse[static_cast<int64_t>(r) * b + lane];
    dam_d[lane] = greedy ? a.dargmax[static_cast<int64_t>(r) * b + lane] : 0;
  }
  __syncwarp();
  // second loads: each node's token in its parent's target row and in the draft row of the parent's depth,
  // and from them, lane-parallel, everything a test needs that does not depend on the walk: p (with the
  // parent's cut) and q of the token, and the node's uniform
  bool bad_tok = false;
  for (int j = lane; j < N; j += kWave) {
    double p0 = 0.0, q = 0.0;
    const int pj = par[j], x = tok[j];
    const bool xok = x >= 0 && x < V;
    if (j > 0 && pj >= 0 && pj < j && xok) {
      const int dep = min(max(kd[pj].y, 0), b - 1);
      if (greedy) {  // p and q one-hot
        p0 = x == am[pj] ? 1.0 : 0.0;
        q = x == dam_d[dep] ? 1.0 : 0.0;
      } else {
        const float l = load_val<DT>(row_ptr(a.tgt, DT, n0 + pj, a.tgt_ld), x);
        const float d = load_val<DDT>(row_ptr(a.draft, DDT, static_cast<int64_t>(r) * b + dep, a.draft_ld), x);
        p0 = l >= cutv[pj] ? exp_tab(static_cast<double>(l) * invT - keptv[pj], etab) : 0.0;
        q = exp_tab(static_cast<double>(d) * invT - dlse_d[dep], etab);
      }
    }
    if (j > 0 && !xok) bad_tok = true;
    pq[j] = make_double2(p0, q);
    uv[j] = j > 0 ? static_cast<float>(u24(philox_at(seed, static_cast<uint32_t>(j - 1), static_cast<uint32_t>(r)).x))
                  : 0.0f;
  }
  if (__ballot(bad_tok) && lane == 0) raise_status(a.status, SV_ST_BAD_TOKEN);
  __syncwarp();
  int u = 0, n = 0;
  double cdraw = 0.0;  // > 0: residual draw at node u with draft row scale cdraw
  bool leaf = false;
  for (;;) {
    const int2 nk = kd[u];
    if (nk.x < 0 || n >= b + (nk.x == 0 ? 1 : 0)) {  // overlapping or stale records
      fail(true);
      return;
    }
    if (nk.x == 0) {
      leaf = true;
      break;
    }
    const size_t zbase = static_cast<size_t>(n0 + u) * (a.max_kids - 1) * a.S;
    double c = 0.0, Z = 1.0;  // the current target: max(0, p - c q) / Z
    int m = 0, next = -1;
    for (int j0 = u + 1; j0 < N && next < 0 && m < nk.x; j0 += kWave) {
      const int j = j0 + lane;
      uint64_t mine = __ballot(j < N && par[min(j, N - 1)] == u);
      while (mine && next < 0) {
        const int jl = __ffsll(static_cast<long long>(mine)) - 1;
        mine &= mine - 1;
        const int jc = j0 + jl;  // the next child in index order
        ++m;
        // greedy: p and q one-hot, and every residual is p again (c stays 0), so each child is tested against p
        const double2 v = pq[jc];
        const double q = v.y;
        const double w = v.x - c * q;
        const double p = c == 0.0 ? v.x : (w > 0.0 ? w / Z : 0.0);
        const double uu = static_cast<double>(uv[jc]);
        const bool accept = q > 0.0 ? uu < p / q : p > 0.0;
        if (lane == 0) {
          if (a.p_out) a.p_out[n0 + jc] = p;
          if (a.q_out) a.q_out[n0 + jc] = q;
          if (a.u_out) a.u_out[n0 + jc] = static_cast<float>(uu);
        }
        if (accept) {
          next = jc;
        } else if (!greedy) {
          // the next target: c_{m+1} = c_m + Z_m (c_1 = 1); a mass emptied by rounding resets it to p
          c = c == 0.0 ? 1.0 : c + Z;
          if (m < nk.x) {
            Z = zsum(a.zpart + zbase + static_cast<size_t>(m - 1) * a.S, a.S);
            if (!(Z > 0.0)) {
              c = 0.0;
              Z = 1.0;
            }
          }
        }
      }
    }
    if (next < 0) {  // every child failed: the residual at u
      cdraw = greedy ? 1.0 : c;
      break;
    }
    if (lane == 0) a.path[static_cast<size_t>(r) * b + n] = next;
    ++n;
    u = next;
  }
  if (lane == 0) {
    a.n_acc[r] = n;
    a.stop_node[r] = u;
    const int g = n0 + u;
    rec.n = u;  // the pick's uniform: word 1 at counter (u, r, 0, 0)
    rec.bonus = leaf ? 1 : 0;
    rec.token = am[u];
    rec.ncorr = 0;
    rec.trow = g;
    rec.drow = static_cast<int64_t>(r) * b + (leaf ? 0 : kd[u].y);
    rec.cut = cutv[u];
    rec.invT = invT;
    rec.kept = keptv[u];
    rec.invTb = 0.0;
    if (greedy) {
      rec.mode = kDrawGreedy;
      rec.dlse = 0.0;
    } else if (leaf || !(cdraw > 0.0)) {
      rec.mode = kDrawP;
      rec.dlse = 0.0;
    } else {
      rec.mode = kDrawResidual;
      rec.dlse = dlse_d[kd[u].y] - log(cdraw);
    }
  }
}

// tree workspace: node records, partial masses, the mass passes' node order
// and per-request child-count histograms (at most max_nodes requests)
struct TreeWs {
  size_t nodes, zpart, order, khist, total;
};

TreeWs tree_ws_layout(int max_nodes, int max_kids, int V) {
  const size_t S = static_cast<size_t>(res_chunks(V)), n = static_cast<size_t>(max_nodes);
  TreeWs l;
  l.nodes = 0;
  l.zpart = align256(sizeof(TreeNode) * n);
  l.order = l.zpart + align256(sizeof(double) * n * (max_kids > 1 ? max_kids - 1 : 1) * S);
  l.khist = l.order + align256(sizeof(int2) * n);
  l.total = l.khist + align256(sizeof(int32_t) * n * (kTreeMaxKids + 1));
  return l;
}

size_t tree_ws_needed(int max_nodes, int max_kids, int V) { return tree_ws_layout(max_nodes, max_kids, V).total; }

}  // namespace sv

using namespace sv;

extern "C" int32_t sv_tree_workspace_bytes(int32_t max_nodes, int32_t max_kids, int32_t V, size_t* out_bytes) {
  if (!out_bytes || max_nodes < 1 || max_kids < 1 || max_kids > kTreeMaxKids || V < 1) return SV_ERR_ARG;
  *out_bytes = tree_ws_needed(max_nodes, max_kids, V);
  return SV_OK;
}

template <int DT, int DDT>
static int32_t launch_tree(const TreeArgs& t, hipStream_t s) {
  for (int k = 1; k < t.max_kids; ++k) {
    hipLaunchKernelGGL((k_tree_mass<DT, DDT>), dim3(kTreeMassGrid), dim3(kTreeNT), 0, s, t, k);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  }
  hipLaunchKernelGGL((k_tree_walk<DT, DDT>), dim3(t.R), dim3(kWave), 0, s, t);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_tree_verify(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                  const int32_t* node_off, const int32_t* parent, const int32_t* token, int32_t R,
                                  int32_t b, int32_t max_nodes, int32_t max_kids, const float* temperature,
                                  const int32_t* row_argmax, const float* row_cut, const double* row_kept_lse,
                                  const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                                  const int32_t* draft_argmax, const double* draft_lse, const uint64_t* seed,
                                  int32_t* n_acc, int32_t* path, int32_t* stop_node, int32_t* token_out,
                                  int32_t* is_bonus, double* p_out, double* q_out, float* u_out, void* ws,
                                  size_t ws_bytes, void* tree_ws, size_t tree_ws_bytes, void* stream) {
  if (!tgt_logits || !node_off || !parent || !token || !temperature || !row_argmax || !row_cut || !row_kept_lse)
    return SV_ERR_ARG;
  if (!draft_logits || !draft_argmax || !draft_lse || !seed || !n_acc || !path || !stop_node || !token_out ||
      !is_bonus || !ws || !tree_ws)
    return SV_ERR_ARG;
  if (R < 1 || R > kTreeMaxReq || b < 1 || b > 64 || V < 1 || max_nodes < R || max_kids < 1 ||
      max_kids > kTreeMaxKids)
    return SV_ERR_ARG;
  if (tgt_ld < V || draft_ld < V) return SV_ERR_ARG;
  if ((dtype != SV_F32 && dtype != SV_BF16) || (draft_dtype != SV_F32 && draft_dtype != SV_BF16)) return SV_ERR_ARG;
  if (!rows_aligned(tgt_logits, dtype, tgt_ld) || !rows_aligned(draft_logits, draft_dtype, draft_ld)) return SV_ERR_ARG;
  if (static_cast<long long>(max_nodes) * res_chunks(V) > 0x7FFFFFFFLL) return SV_ERR_ARG;
  const WsLayout l = ws_layout(R, b, 0, V);
  if (ws_bytes < l.total || tree_ws_bytes < tree_ws_needed(max_nodes, max_kids, V)) return SV_ERR_WORKSPACE;
  TreeArgs t{};
  t.tgt = tgt_logits; t.dtype = dtype; t.tgt_ld = tgt_ld; t.V = V;
  t.node_off = node_off; t.parent = parent; t.token = token;
  t.R = R; t.b = b; t.max_nodes = max_nodes; t.max_kids = max_kids; t.S = res_chunks(V);
  t.T = temperature; t.row_argmax = row_argmax; t.row_cut = row_cut; t.row_kept = row_kept_lse;
  t.draft = draft_logits; t.ddtype = draft_dtype; t.draft_ld = draft_ld; t.dargmax = draft_argmax; t.dlse = draft_lse;
  t.seed = seed; t.n_acc = n_acc; t.path = path; t.stop_node = stop_node;
  t.p_out = p_out; t.q_out = q_out; t.u_out = u_out;
  const TreeWs tl = tree_ws_layout(max_nodes, max_kids, V);
  char* twb = static_cast<char*>(tree_ws);
  t.nodes = reinterpret_cast<TreeNode*>(twb + tl.nodes);
  t.zpart = reinterpret_cast<double*>(twb + tl.zpart);
  t.order = reinterpret_cast<int2*>(twb + tl.order);
  t.khist = reinterpret_cast<int32_t*>(twb + tl.khist);
  t.rec = reinterpret_cast<DrawRec*>(static_cast<char*>(ws) + l.rec);
  t.status = status_word(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_tree_prep, dim3(R), dim3(kTreeNT), 0, s, t);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  const bool t16 = dtype == SV_BF16, d16 = draft_dtype == SV_BF16;
  const int32_t st = t16 ? (d16 ? launch_tree<SV_BF16, SV_BF16>(t, s) : launch_tree<SV_BF16, SV_F32>(t, s))
                         : (d16 ? launch_tree<SV_F32, SV_BF16>(t, s) : launch_tree<SV_F32, SV_F32>(t, s));
  if (st != SV_OK) return st;
  // the draw from the walk's records (dense weights max(0, p - c q))
  SampleArgs a{};
  a.tgt = tgt_logits; a.dtype = dtype; a.tgt_ld = tgt_ld; a.V = V; a.R = R; a.b = b; a.T = temperature;
  a.q_mode = SV_Q_DENSE; a.draft = draft_logits; a.ddtype = draft_dtype; a.draft_ld = draft_ld; a.seed = seed;
  a.token = token_out; a.is_bonus = is_bonus; a.status = status_word(ws);
  a.rec = t.rec;
  a.sub = reinterpret_cast<double*>(static_cast<char*>(ws) + l.sub);
  a.NSUB = sub_chunks(V);
  a.S = res_chunks(V);
  return launch_record_draw(a, s);
}
