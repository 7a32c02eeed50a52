// Rotary positions inside the working context (InfLLM Guide, "Operational
// Checklist", RoPE item: the native base is kept and memory units take
// local relative offsets).
//
// q and k arrive turned by RoPE at their absolute positions (rotate-half
// pairs (c, c + D/2), angle p * theta^(-2c/D)).  For the chunk whose first
// query is at t0 let lo = max(n_init, t0 - W + 1); every token gets a place
// in the working context:
//     initial token p < n_init            -> p
//     key p of the unit in sel slot m     -> n_init + m*B + (p - jB)
//                                            (jB: first position of its block)
//     token p >= lo (window keys, queries) -> n_init + k_m*B + (p - lo)
// Turning q from t to its place and k from p to its place gives the logit
// q . R(s_k - s_q) k, where s = place - position.  Window keys and queries
// share s = n_init + k_m*B - lo, so the window needs nothing; an initial
// token turns by -E_s and a unit key by -E_m with
//     E_s = n_init + k_m*B - lo,      E_m = (k_m - m)*B + jB - lo,
// and a query before n_init (its own place is its position) turns by -E_s
// too (it sees initial tokens only).  Shifts are whole positions below
// 2^31; angles are reduced to one turn in fp64 before the fp32 sine and
// cosine, so their error does not grow with the position.
#pragma once

#include "common.h"

namespace infllm {

// DPP row_ror:8: lane i of each 16-lane row reads lane (i + 8) % 16 -- with
// the columns of a head spread over 16 lanes, the lane holding the partner
// half (c <-> c + D/2).
#define INFLLM_DPP_ROR8 0x128

constexpr double kTwoPi = 6.283185307179586;

// Frequency i of a head of size D, in turns per position: theta^(-2i/D) / 2pi.
__device__ __forceinline__ double rope_turns(double theta, int D, int i) {
  return pow(theta, -2.0 * (double)i / (double)D) * (1.0 / kTwoPi);
}

// cos and sin of E positions at frequency f (turns per position).  The
// angle is reduced in fp64 to a quarter turn q plus a remainder a with
// |a| <= pi/4; sin a and cos a are their Taylor series through a^9 and a^10
// (truncation below 2e-9 there), evaluated in fp32, and the quarter turns
// are applied exactly: sin(q pi/2 + a), cos(q pi/2 + a) are (sin a, cos a),
// (cos a, -sin a), (-sin a, -cos a), (-cos a, sin a) for q = 0, 1, 2, 3.
__device__ __forceinline__ void rope_cs(int E, double f, float* c, float* s) {
  double x = (double)E * f;
  x -= rint(x);                        // turns, within half a turn
  const double r = 4.0 * x, qd = rint(r);
  const float a = (float)((r - qd) * (0.25 * kTwoPi)), a2 = a * a;
  const float sa =
      a * fmaf(a2, fmaf(a2, fmaf(a2, fmaf(a2, 1.f / 362880.f, -1.f / 5040.f), 1.f / 120.f),
                        -1.f / 6.f), 1.f);
  const float ca = fmaf(
      a2, fmaf(a2, fmaf(a2, fmaf(a2, fmaf(a2, -1.f / 3628800.f, 1.f / 40320.f), -1.f / 720.f),
                        1.f / 24.f), -0.5f), 1.f);
  const int q = (int)qd & 3;
  *s = q == 0 ? sa : (q == 1 ? ca : (q == 2 ? -sa : -ca));
  *c = q == 0 ? ca : (q == 1 ? -sa : (q == 2 ? -ca : sa));
}

// First place of the local run for the chunk starting at t0.
__device__ __forceinline__ int64_t rope_local_start(int64_t t0, int n_init, int W) {
  const int64_t a = t0 - W + 1;
  return a > n_init ? a : n_init;
}

// Turn by -E of one lane's columns: x holds n columns of the lower (low =
// true) or upper half, partner the same columns of the other half;
// c, s = cos and sin of E at those columns' frequencies.
__device__ __forceinline__ float rope_turn(float x, float partner, float c, float s, bool low) {
  return fmaf(partner, low ? s : -s, x * c);
}

}  // namespace infllm
