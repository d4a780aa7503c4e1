// The fused vocabulary-wide acceptance step.
//
// row_stats: one block per (row, 4096-logit chunk) streams the chunk once (coalesced) and
// records its max, lowest argmax and s_c = sum exp((l - m_c)/T) in double.
// decide: one block per slot combines the chunk statistics of the rows it needs
// (m = max m_c, S = sum s_c exp((m_c - m)/T)) and runs the slot's decisions:
//   p(x) = exp((l_x - m)/T) / S; acceptance u < p(x)/q(x) (q from the previous pass's
//   MASK row, or 1 for an argmax proposal); on the first rejection a draw from
//   normalize(max(0, p - q)) (p with x removed for an argmax proposal; p itself when the
//   residual has no mass); otherwise z_1 from the last verified row and the proposals of
//   the MASK rows.  A categorical draw finds the chunk whose prefix crosses u*S from the
//   chunk sums, then re-reads only that chunk (two-level inverse CDF).
// The method (wiki note "Introspective Diffusion Language Models", Key claims and Method;
// Agentic Commons post, "How Introspective Strided Decoding Works"): acceptance
// min(1, p/q) with p the anchor of the current pass and q the proposal distribution of the
// previous pass, first rejection restarts the block, logit shift makes the first new token
// always accepted.
#include <float.h>

#include "isd_common.h"

namespace isd {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int NT = 256;
constexpr int PER = kStatChunk / NT;   // logits per thread in a chunk

__global__ __launch_bounds__(NT) void row_stats_kernel(const float* logits, int V, float T, ChunkStat* stats,
                                                       int n_chunks, const int32_t* m_live) {
  __shared__ float shm[4], shm2[4];
  __shared__ int sha[4];
  __shared__ double shs[4];
  __shared__ int shbad[4];
  const int row = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  if (m_live && row >= *m_live) return;              // a dead row of a packed pass
  const int c0 = c * kStatChunk, c1 = min(V, c0 + kStatChunk);
  const float* l = logits + (size_t)row * V;
  float v[PER];
  float mx = kNegInf, mx2 = kNegInf;   // largest and second largest (a repeated maximum counts twice)
  int am = INT_MAX;
  int bad = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = c0 + tid + NT * k;
    const float x = j < c1 ? l[j] : kNegInf;
    v[k] = x;
    if (j < c1 && !isfinite(x)) bad = 1;
    mx2 = fmaxf(mx2, fminf(mx, x));
    if (x > mx) {
      mx = x;
      am = j;
    }
  }
  // (max, lowest index) reduction; the second largest of two (max, second) pairs is the larger
  // of the smaller maximum and the two seconds
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64);
    const float s2 = __shfl_xor(mx2, o, 64);
    const int a2 = __shfl_xor(am, o, 64);
    mx2 = fmaxf(fminf(mx, m2), fmaxf(mx2, s2));
    if (m2 > mx || (m2 == mx && a2 < am)) {
      mx = m2;
      am = a2;
    }
  }
  bad = __any(bad) ? 1 : 0;
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    shm[w] = mx;
    shm2[w] = mx2;
    sha[w] = am;
    shbad[w] = bad;
  }
  __syncthreads();
  mx = shm[0];
  mx2 = shm2[0];
  am = sha[0];
  for (int i = 1; i < 4; ++i) {
    mx2 = fmaxf(fminf(mx, shm[i]), fmaxf(mx2, shm2[i]));
    if (shm[i] > mx || (shm[i] == mx && sha[i] < am)) {
      mx = shm[i];
      am = sha[i];
    }
  }
  bad = shbad[0] | shbad[1] | shbad[2] | shbad[3];
  double s = 0.0;
  if (T > 0.f && !bad) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = c0 + tid + NT * k;
      if (j < c1) s += (double)expf((v[k] - mx) / T);
    }
    s = wave_sum_d(s);
    if ((tid & 63) == 0) shs[w] = s;
    __syncthreads();
    s = (shs[0] + shs[1]) + (shs[2] + shs[3]);
  }
  if (tid == 0) {
    ChunkStat cs;
    cs.m = bad ? __builtin_nanf("") : mx;
    cs.m2 = mx2;
    cs.arg = am;
    cs.pad = 0;
    cs.s = s;
    stats[(size_t)row * n_chunks + c] = cs;
  }
}

// ----------------------------------------------------------------------------- decide
struct Smem {
  double d[NT];
  int i[NT];
  float f[4], f2[4];
  double dw[4];
  int iw[4];
  double margin;      // margin of the last categorical draw
};

__device__ double bsum(double v, Smem& sm) {
  v = wave_sum_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.dw[threadIdx.x >> 6] = v;
  __syncthreads();
  return (sm.dw[0] + sm.dw[1]) + (sm.dw[2] + sm.dw[3]);
}

__device__ int bmin_i(int v, Smem& sm) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.iw[threadIdx.x >> 6] = v;
  __syncthreads();
  return min(min(sm.iw[0], sm.iw[1]), min(sm.iw[2], sm.iw[3]));
}

__device__ int bmax_i(int v, Smem& sm) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm.iw[threadIdx.x >> 6] = v;
  __syncthreads();
  return max(max(sm.iw[0], sm.iw[1]), max(sm.iw[2], sm.iw[3]));
}

// Inclusive prefix sum of one double per thread (Hillis-Steele in LDS).
__device__ double bscan(double v, Smem& sm) {
  const int tid = threadIdx.x;
  __syncthreads();
  sm.d[tid] = v;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const double t = tid >= off ? sm.d[tid - off] : 0.0;
    __syncthreads();
    sm.d[tid] += t;
    __syncthreads();
  }
  return sm.d[tid];
}

struct RowStat {
  float m, m2;        // largest and second largest logit
  int arg;
  double S;
  bool ok;
};

// Combine the chunk statistics of one row: m = max m_c (lowest argmax), S = sum s_c e^{(m_c-m)/T}.
__device__ RowStat row_stat(const ChunkStat* cs, int nc, float T, Smem& sm) {
  float m = kNegInf, sec = kNegInf;
  int a = INT_MAX;
  bool bad = false;
  for (int c = threadIdx.x; c < nc; c += NT) {
    const ChunkStat x = cs[c];
    if (!isfinite(x.m)) bad = true;
    sec = fmaxf(fminf(m, x.m), fmaxf(sec, x.m2));
    if (x.m > m || (x.m == m && x.arg < a)) {
      m = x.m;
      a = x.arg;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(sec, o, 64);
    const int a2 = __shfl_xor(a, o, 64);
    sec = fmaxf(fminf(m, m2), fmaxf(sec, s2));
    if (m2 > m || (m2 == m && a2 < a)) {
      m = m2;
      a = a2;
    }
  }
  const int nbad = bmax_i(bad ? 1 : 0, sm);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sm.f[threadIdx.x >> 6] = m;
    sm.f2[threadIdx.x >> 6] = sec;
    sm.iw[threadIdx.x >> 6] = a;
  }
  __syncthreads();
  m = sm.f[0];
  sec = sm.f2[0];
  a = sm.iw[0];
  for (int i = 1; i < 4; ++i) {
    sec = fmaxf(fminf(m, sm.f[i]), fmaxf(sec, sm.f2[i]));
    if (sm.f[i] > m || (sm.f[i] == m && sm.iw[i] < a)) {
      m = sm.f[i];
      a = sm.iw[i];
    }
  }
  RowStat r;
  r.m = m;
  r.m2 = sec;
  r.arg = a;
  r.S = 0.0;
  if (T > 0.f) {
    double s = 0.0;
    for (int c = threadIdx.x; c < nc; c += NT) s += cs[c].s * exp(((double)cs[c].m - (double)m) / (double)T);
    r.S = bsum(s, sm);
  }
  r.ok = !nbad && isfinite(m) && (T == 0.f || (isfinite(r.S) && r.S > 0.0));
  return r;
}

ISD_DEV double weight_of(float l, float m, float T) { return (double)expf((l - m) / T); }

// Margin of a draw (left in sm.margin for every thread): the distance of the target u*S to the
// nearest edge [lo, lo + w) of the chosen token's interval, divided by S; 0 for a fallback.
__device__ void publish_margin(int j, int cand, double lo, double w, double target, double total, Smem& sm) {
  __syncthreads();
  if (threadIdx.x == 0) sm.margin = 0.0;
  __syncthreads();
  if (cand == j && cand != INT_MAX) sm.margin = fmin(target - lo, lo + w - target) / total;
  __syncthreads();
}

// Smallest j with (prefix of w up to j) > target, w_j = exp((l_j - m)/T) with w_excl = 0;
// chunk weights cw (one per chunk, excl removed) locate the chunk first.  total: the sum of
// the weights (target = u * total).
__device__ int cat_in_row(const float* l, int V, int nc, const double* cw_in, float m, float T, double target,
                          double total, int excl, Smem& sm) {
  const int tid = threadIdx.x;
  // chunk level (nc <= NT)
  const double cw = tid < nc ? cw_in[tid] : 0.0;
  const double P = bscan(cw, sm);
  int cstar = bmin_i((tid < nc && P > target) ? tid : INT_MAX, sm);
  if (cstar == INT_MAX) cstar = bmax_i((tid < nc && cw > 0.0) ? tid : -1, sm);
  if (cstar < 0) return excl == 0 ? 1 : 0;   // no mass anywhere (callers guard against this)
  __syncthreads();
  if (tid == cstar) sm.dw[0] = P - cw;
  __syncthreads();
  const double base = sm.dw[0];
  // element level inside chunk cstar: thread t owns PER consecutive logits
  const int j0 = cstar * kStatChunk + tid * PER;
  double wv[PER];
  double tsum = 0.0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = j0 + k;
    const float lj = l[min(j, V - 1)];   // unconditional load (past the row: counted as zero)
    const double w = (j < V && j != excl) ? weight_of(lj, m, T) : 0.0;
    wv[k] = w;
    tsum += w;
  }
  const double excl_pref = bscan(tsum, sm) - tsum;
  double run = base + excl_pref;
  int cand = INT_MAX, lastpos = -1;
  double cand_lo = 0.0, cand_w = 0.0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const double lo = run;
    run += wv[k];
    if (wv[k] > 0.0) lastpos = j0 + k;
    if (cand == INT_MAX && wv[k] > 0.0 && run > target) {
      cand = j0 + k;
      cand_lo = lo;
      cand_w = wv[k];
    }
  }
  int j = bmin_i(cand, sm);
  if (j == INT_MAX) j = bmax_i(lastpos, sm);
  publish_margin(j, cand, cand_lo, cand_w, target, total, sm);
  return j;
}

struct Decider {
  const SampleArgs& a;
  Smem& sm;
  int nc;

  __device__ RowStat stat_cur(int row) { return row_stat(a.stats + (size_t)row * nc, nc, a.T, sm); }
  __device__ RowStat stat_prev(int row) { return row_stat(a.q_stats + (size_t)row * nc, nc, a.T, sm); }

  // chunk weights of a row relative to its max, with token `excl` removed
  __device__ void chunk_weights(const ChunkStat* cs, const float* l, const RowStat& rs, int excl) {
    __syncthreads();
    if (threadIdx.x < nc) {
      double w = cs[threadIdx.x].s * exp(((double)cs[threadIdx.x].m - (double)rs.m) / (double)a.T);
      if (excl >= 0 && excl / kStatChunk == (int)threadIdx.x) w = fmax(0.0, w - weight_of(l[excl], rs.m, a.T));
      sm.d[threadIdx.x] = w;
    }
    __syncthreads();
  }

  // Cat(softmax_T(row), u), excluding `excl` (argmax-proposal residual) when >= 0
  __device__ int draw(int row, const RowStat& rs, double u, int excl) {
    const float* l = a.logits + (size_t)row * a.V;
    const ChunkStat* cs = a.stats + (size_t)row * nc;
    __shared__ double cw[NT];
    chunk_weights(cs, l, rs, excl);
    if (threadIdx.x < NT) cw[threadIdx.x] = threadIdx.x < nc ? sm.d[threadIdx.x] : 0.0;
    __syncthreads();
    double tot = bsum(threadIdx.x < nc ? cw[threadIdx.x] : 0.0, sm);
    if (!(tot > 0.0)) {   // residual without mass: fall back to p itself
      chunk_weights(cs, l, rs, -1);
      if (threadIdx.x < NT) cw[threadIdx.x] = threadIdx.x < nc ? sm.d[threadIdx.x] : 0.0;
      __syncthreads();
      tot = bsum(threadIdx.x < nc ? cw[threadIdx.x] : 0.0, sm);
      excl = -1;
    }
    return cat_in_row(l, a.V, nc, cw, rs.m, a.T, u * tot, tot, excl, sm);
  }

  // normalize(max(0, p - q)) with q the previous pass's row qrow.  One sweep over the row
  // gives every chunk's residual mass (each wave sums its share of a chunk, no block barrier
  // per chunk; the four wave sums are added in a fixed order), then the chunk the draw lands
  // in is re-read element by element.
  __device__ int resid_draw(int row, const RowStat& ps, int qrow, const RowStat& qs, double u) {
    const float* lp = a.logits + (size_t)row * a.V;
    const float* lq = a.q_logits + (size_t)qrow * a.V;
    __shared__ double rc[NT];
    __shared__ double rcw[NT / 64][NT];
    const int tid = threadIdx.x;
    const double ips = 1.0 / ps.S, iqs = 1.0 / qs.S;
    // j past the row reads its last element and counts zero: the loads carry no condition, so
    // all of a thread's loads of a chunk are in flight together
    auto resid = [&](int j) {
      const int jj = min(j, a.V - 1);
      const double r = weight_of(lp[jj], ps.m, a.T) * ips - weight_of(lq[jj], qs.m, a.T) * iqs;
      return (j < a.V && r > 0.0) ? r : 0.0;
    };
    for (int c = 0; c < nc; ++c) {
      double s = 0.0;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        s += resid(c * kStatChunk + tid + NT * k);
      }
      s = wave_sum_d(s);
      if ((tid & 63) == 0) rcw[tid >> 6][c] = s;
    }
    __syncthreads();
    if (tid < nc) rc[tid] = (rcw[0][tid] + rcw[1][tid]) + (rcw[2][tid] + rcw[3][tid]);
    __syncthreads();
    const double tot = bsum(tid < nc ? rc[tid] : 0.0, sm);
    if (!(tot > 0.0)) return draw(row, ps, u, -1);
    // chunk level
    const double cwv = tid < nc ? rc[tid] : 0.0;
    const double P = bscan(cwv, sm);
    const double target = u * tot;
    int cstar = bmin_i((tid < nc && P > target) ? tid : INT_MAX, sm);
    if (cstar == INT_MAX) cstar = bmax_i((tid < nc && cwv > 0.0) ? tid : -1, sm);
    __syncthreads();
    if (tid == cstar) sm.dw[0] = P - cwv;
    __syncthreads();
    const double base = sm.dw[0];
    const int j0 = cstar * kStatChunk + tid * PER;
    double wv[PER];
    double tsum = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = j0 + k;
      wv[k] = resid(j);
      tsum += wv[k];
    }
    const double excl_pref = bscan(tsum, sm) - tsum;
    double run = base + excl_pref;
    int cand = INT_MAX, lastpos = -1;
    double cand_lo = 0.0, cand_w = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const double lo = run;
      run += wv[k];
      if (wv[k] > 0.0) lastpos = j0 + k;
      if (cand == INT_MAX && wv[k] > 0.0 && run > target) {
        cand = j0 + k;
        cand_lo = lo;
        cand_w = wv[k];
      }
    }
    int j = bmin_i(cand, sm);
    if (j == INT_MAX) j = bmax_i(lastpos, sm);
    publish_margin(j, cand, cand_lo, cand_w, target, tot, sm);
    return j;
  }
};

__global__ __launch_bounds__(NT) void decide_kernel(SampleArgs a) {
  __shared__ Smem sm;
  __shared__ int s_tok[2 * ISD_MAX_STRIDE];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int b = a.slot_ids ? a.slot_ids[i] : i;
  isd_slot* st = &a.slots[b];
  const int N = a.N;
  Decider D{a, sm, a.n_chunks};
  const bool greedy = !(a.T > 0.f);

  if (a.prefill) {
    if (st->state != ISD_SLOT_B) {     // finished at admission (no KV pages on the device)
      if (tid == 0) a.first_tok[i] = -1;
      return;
    }
    const RowStat rs = D.stat_cur(i);
    int z = 0;
    if (rs.ok) {
      if (greedy) z = rs.arg;
      else z = D.draw(i, rs, philox_uniform(a.seed, b, 0, st->L, 1), -1);
    }
    __syncthreads();
    if (tid == 0) {
      if (!rs.ok) {
        st->status = ISD_E_NONFINITE;
        st->state = ISD_SLOT_DONE;
        a.first_tok[i] = -1;
      } else {
        st->c = z;
        st->n_gen = 1;
        st->t = 1;
        st->committed = 1;
        if (st->n_gen >= st->max_new) st->state = ISD_SLOT_DONE;
        a.first_tok[i] = z;
      }
    }
    return;
  }

  const int state = st->state;
  if (state != ISD_SLOT_A && state != ISD_SLOT_B) {
    if (tid < N) a.tokens[(size_t)b * N + tid] = -1;
    if (tid < 2 * N) {
      if (a.margins) a.margins[(size_t)b * 2 * N + tid] = -1.0;
      if (a.kinds) a.kinds[(size_t)b * 2 * N + tid] = -1;
    }
    if (tid == 0) {
      a.n_commit[b] = 0;
      a.n_accept[b] = 0;
    }
    return;
  }
  const int R = a.rows_per_slot, base_row = a.row_off ? a.row_off[b] : b * R;
  const int L = st->L, t = st->t;
  int ncommit = 0, nacc = 0, nver = 0;
  // debug record: kind and margin of each decision in order (an argmax decision's margin is
  // the top-2 logit gap of its row)
  int nd = 0;
  auto note = [&](int kind, double margin) {
    if (tid == 0) {
      if (a.margins) a.margins[(size_t)b * 2 * N + nd] = margin;
      if (a.kinds) a.kinds[(size_t)b * 2 * N + nd] = kind;
    }
    ++nd;
  };
  auto gap = [](const RowStat& r) { return (double)r.m - (double)r.m2; };
  double msum = 0.0;                   // meter: acceptance probabilities of the pending tokens
  bool failed = false;
  int newL = L, newc = st->c, newstate = ISD_SLOT_A;
  int npend = 0;
  int pend[ISD_MAX_STRIDE], qrow[ISD_MAX_STRIDE];

  auto commit = [&](int tok) {
    if (tid == 0) s_tok[ncommit] = tok;
    ++ncommit;
  };
  auto propose_from = [&](int row, int pos) {
    const RowStat rs = D.stat_cur(row);
    if (!rs.ok) {
      failed = true;
      return;
    }
    int z;
    int qr = -1;
    if (greedy || a.propose == ISD_PROPOSE_ARGMAX) {
      z = rs.arg;
      note(ISD_DEC_PROPOSE, gap(rs));
    } else {
      z = D.draw(row, rs, philox_uniform(a.seed, b, t, pos, 1), -1);
      note(ISD_DEC_PROPOSE, sm.margin);
      qr = row;
    }
    pend[npend] = z;
    qrow[npend] = qr;
    ++npend;
  };

  bool rejected = false;
  if (state == ISD_SLOT_A) {
    for (int k = 1; k < N && !failed; ++k) {
      const int row = base_row + k - 1;
      const int v = st->pending[k - 1];
      const RowStat ps = D.stat_cur(row);
      const int qr = st->q_row[k - 1];
      if (!ps.ok || v < 0 || v >= a.V || qr >= a.q_rows) {
        failed = true;
        break;
      }
      ++nver;
      bool ok;
      RowStat qs;
      qs.ok = true;
      // q is the proposing row's distribution for a sampled proposal, delta(v) for an argmax one
      const bool sampled_q = a.propose == ISD_PROPOSE_SAMPLE && qr >= 0 && a.q_logits;
      if (greedy) {
        ok = (v == ps.arg);
        if (a.meter) {
          msum += ok ? 1.0 : 0.0;
          ok = true;
        }
        note(ISD_DEC_ACCEPT, a.meter ? __builtin_huge_val() : gap(ps));
      } else {
        const double px = weight_of(a.logits[(size_t)row * a.V + v], ps.m, a.T) / ps.S;
        double qx = 1.0;
        if (sampled_q) {
          qs = D.stat_prev(qr);
          if (!qs.ok) {
            failed = true;
            break;
          }
          qx = weight_of(a.q_logits[(size_t)qr * a.V + v], qs.m, a.T) / qs.S;
        }
        if (a.meter) {
          msum += fmin(1.0, px / qx);
          ok = true;
          note(ISD_DEC_ACCEPT, __builtin_huge_val());
        } else {
          const double u = philox_uniform(a.seed, b, t, L + k, 0);
          ok = u < px / qx;
          note(ISD_DEC_ACCEPT, fabs(u - fmin(1.0, px / qx)));
        }
      }
      if (ok) {
        commit(v);
        ++nacc;
        continue;
      }
      int r;
      if (greedy) {
        r = ps.arg;
        note(ISD_DEC_RESID, gap(ps));
      } else {
        const double u2 = philox_uniform(a.seed, b, t, L + k, 1);
        if (sampled_q) r = D.resid_draw(row, ps, qr, qs, u2);
        else r = D.draw(row, ps, u2, v);
        note(ISD_DEC_RESID, sm.margin);
      }
      commit(r);
      rejected = true;
      newL = L + k;
      newc = r;
      newstate = ISD_SLOT_B;
      break;
    }
    if (!rejected && !failed) {
      const int row = base_row + N - 1;
      const RowStat rs = D.stat_cur(row);
      if (!rs.ok) {
        failed = true;
      } else {
        const int z1 = greedy ? rs.arg : D.draw(row, rs, philox_uniform(a.seed, b, t, L + N, 1), -1);
        note(ISD_DEC_Z1, greedy ? gap(rs) : sm.margin);
        commit(z1);
        for (int j = 1; j < N && !failed; ++j) propose_from(base_row + N - 1 + j, L + N + j);
        newL = L + N;
        newc = z1;
        newstate = ISD_SLOT_A;
      }
    }
  } else {
    const RowStat rs = D.stat_cur(base_row);
    if (!rs.ok) {
      failed = true;
    } else {
      const int z1 = greedy ? rs.arg : D.draw(base_row, rs, philox_uniform(a.seed, b, t, L + 1, 1), -1);
      note(ISD_DEC_Z1, greedy ? gap(rs) : sm.margin);
      commit(z1);
      for (int j = 1; j < N && !failed; ++j) propose_from(base_row + j, L + 1 + j);
      newL = L + 1;
      newc = z1;
      newstate = ISD_SLOT_A;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (failed) {
      st->status = ISD_E_NONFINITE;
      st->state = ISD_SLOT_DONE;
      ncommit = 0;
    } else {
      const int room = st->max_new - st->n_gen;
      if (ncommit > room) ncommit = room;
      st->n_gen += ncommit;
      st->L = newL;
      st->c = newc;
      st->state = newstate;
      for (int j = 0; j < ISD_MAX_STRIDE - 1; ++j) {
        st->pending[j] = (newstate == ISD_SLOT_A && j < npend) ? pend[j] : -1;
        st->q_row[j] = (newstate == ISD_SLOT_A && j < npend) ? qrow[j] : -1;
      }
      if (st->n_gen >= st->max_new) st->state = ISD_SLOT_DONE;
    }
    st->t = t + 1;
    st->passes += 1;
    st->verified += nver;
    st->accepted += nacc;
    if (a.meter) {
      st->meter_sum += msum;
      st->meter_n += nver;
    }
    st->committed += ncommit;
    for (int k = 0; k < N; ++k) a.tokens[(size_t)b * N + k] = k < ncommit ? s_tok[k] : -1;
    a.n_commit[b] = ncommit;
    a.n_accept[b] = nacc;
    if (failed) nd = 0;                        // a failed pass took no decision
    for (int k = nd; k < 2 * N; ++k) {
      if (a.margins) a.margins[(size_t)b * 2 * N + k] = -1.0;
      if (a.kinds) a.kinds[(size_t)b * 2 * N + k] = -1;
    }
  }
}

}  // namespace

hipError_t launch_row_stats(const float* logits, int rows, int V, float T, ChunkStat* stats, hipStream_t s,
                            const int32_t* m_live) {
  if (rows <= 0) return hipSuccess;
  const int nc = (V + kStatChunk - 1) / kStatChunk;
  hipLaunchKernelGGL(row_stats_kernel, dim3(rows, nc), dim3(NT), 0, s, logits, V, T, stats, nc, m_live);
  return hipGetLastError();
}

hipError_t launch_decide(const SampleArgs& a, hipStream_t s) {
  if (a.n_slots <= 0) return hipSuccess;
  if (a.n_chunks > NT) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decide_kernel, dim3(a.n_slots), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace isd
