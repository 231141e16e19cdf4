// Where the pieces of a split segment store their partials, and how many
// there are.  Shared by the decode kernels (the workgroup that counts a
// segment's last piece walks its slots to merge them) and a host-compiled
// test that checks them against brute-force ownership; plain integer
// arithmetic, nothing device-specific.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// the split-K decode, whose partial results are merged by log-sum-exp.
#pragma once

namespace pkv {

// Fixed partitions p_lo .. p_hi of one segment, at slots base + p.
struct SplitSlots {
  int base, p_lo, p_hi;
  __host__ __device__ int count() const { return p_hi - p_lo + 1; }
  __host__ __device__ bool slot(int k, int& s) const {
    s = base + p_lo + k;
    return true;
  }
};

// Balanced split: W units over N workgroups, workgroup w taking
// [w W / N, (w+1) W / N).  Every segment's real units [S, E) are preceded by
// cost units starting at Sv (S - Sv stands for a piece's fixed cost).  The
// pieces of the segment are the workgroups whose ranges meet [S, E).  With
// W > N every range holds at least one unit, so they are w_first .. w_last.
// With W <= N a range holds one unit or none, and the workgroups with an
// empty range (which store nothing and never count in) lie between those;
// the pieces are then the owners of units S .. E - 1, one each.  A
// workgroup meets at most two split segments, the one its range starts in
// and the one it ends in: a range that starts at or after Sv met the segment
// first (slot 2 w), otherwise second (slot 2 w + 1).
struct BalancedSlots {
  long long W, S, E, Sv;
  int N, w_first, w_last;
  __host__ __device__ BalancedSlots(long long W_, long long S_, long long E_, long long Sv_, int N_)
      : W(W_), S(S_), E(E_), Sv(Sv_), N(N_) {
    w_first = (int)(((S + 1) * N - 1) / W);
    w_last = (int)((E * N - 1) / W);
  }
  __host__ __device__ int count() const { return W <= N ? (int)(E - S) : w_last - w_first + 1; }
  __host__ __device__ bool slot(int k, int& s) const {
    const int w = W <= N ? (int)(((S + k + 1) * N - 1) / W) : w_first + k;
    const long long a0 = (long long)w * W / N;
    s = a0 < Sv ? 2 * w + 1 : 2 * w;
    return true;
  }
};

// Persistent split-K: I items (partitions of all segments, segment after
// segment) over N workgroups, workgroup w taking [w I / N, (w+1) I / N).
// The pieces of a segment's items [S, E) are the workgroups whose ranges
// meet them, each storing one partial at the slot of its first partition in
// the segment (base + its first item - S).  With I <= N a range holds one
// item or none, and the pieces are the owners of items S .. E - 1.
struct RunSlots {
  long long I, S, E;
  int N, base, w_first, w_last;
  __host__ __device__ RunSlots(long long I_, long long S_, long long E_, int N_, int base_)
      : I(I_), S(S_), E(E_), N(N_), base(base_) {
    w_first = (int)(((S + 1) * N - 1) / I);
    w_last = (int)((E * N - 1) / I);
  }
  __host__ __device__ int count() const { return I <= N ? (int)(E - S) : w_last - w_first + 1; }
  __host__ __device__ bool slot(int k, int& s) const {
    const int w = I <= N ? (int)(((S + k + 1) * N - 1) / I) : w_first + k;
    const long long start = (long long)w * I / N;
    const long long first = S < start ? start : S;
    s = base + (int)(first - S);
    return true;
  }
};

}  // namespace pkv
