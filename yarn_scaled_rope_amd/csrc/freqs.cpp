// Host-side rotary frequency table and logit temperature (yarn_rope_freqs).
//
// "Arch 03 -- Long Context" slide deck: RoPE slide (theta_i = base^(-2i/d)),
// Position Interpolation slide (theta_i / s), NTK-aware slide (base raised to
// base * s^(d/(d-2))), YaRN slide and steps table (wavelength
// lambda_i = 2 pi / theta_i, alpha = 1, beta = 32, temperature
// t = 0.1 ln s + 1).  The YaRN ramp runs over the number of turns a pair makes
// across the original context, r_i = L / lambda_i: at or above beta the pair is
// left unscaled, at or below alpha it is interpolated like PI, linear between.
//
// Everything is computed in double and each fp32 entry is the round-to-
// nearest-even of its double value.  Pure regions are assigned directly, so
// s = 1 reproduces the plain table bit for bit.
#include <cmath>
#include <cstdio>

#include "yarnattn.h"
#include "yr_internal.h"

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

double plain_theta(int i, int d, double base) {
  return std::pow(base, -2.0 * (double)i / (double)d);
}

}  // namespace

extern "C" int yarn_rope_freqs(int head_dim, double base, double factor,
                               long long original_max_position, double alpha,
                               double beta, int method, float *inv_freq_f32,
                               double *inv_freq_f64, double *attn_factor) {
  if (head_dim < 2 || head_dim > 1024 || (head_dim & 1))
    return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: head_dim must be even and in [2, 1024]");
  if (!std::isfinite(base) || !(base > 1.0))
    return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: base must be finite and > 1");
  if (method != YR_ROPE_PLAIN && method != YR_ROPE_PI && method != YR_ROPE_NTK &&
      method != YR_ROPE_YARN)
    return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: unknown method");
  if (method == YR_ROPE_NTK && head_dim < 4)
    return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: NTK-aware scaling needs head_dim >= 4 "
                                    "(the base is raised to s^(d/(d-2)))");
  if (method != YR_ROPE_PLAIN && (!std::isfinite(factor) || !(factor >= 1.0)))
    return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: factor s must be finite and >= 1");
  if (method == YR_ROPE_YARN) {
    if (original_max_position < 1)
      return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: original_max_position must be >= 1");
    if (!std::isfinite(alpha) || !std::isfinite(beta) || !(alpha >= 0.0) || !(alpha < beta))
      return yr::fail(YR_ERR_INVALID, "yarn_rope_freqs: need 0 <= alpha < beta");
  }

  const int half = head_dim / 2;
  double eff_base = base;
  if (method == YR_ROPE_NTK)
    eff_base = base * std::pow(factor, (double)head_dim / ((double)head_dim - 2.0));

  for (int i = 0; i < half; ++i) {
    const double th = plain_theta(i, head_dim, eff_base);
    double out = th;
    if (method == YR_ROPE_PI) {
      out = th / factor;
    } else if (method == YR_ROPE_YARN) {
      const double turns = (double)original_max_position * th / kTwoPi;  // L / lambda
      const double pi_th = th / factor;
      if (turns <= alpha) {
        out = pi_th;
      } else if (turns >= beta) {
        out = th;
      } else {
        const double gamma = (turns - alpha) / (beta - alpha);
        out = pi_th + gamma * (th - pi_th);
      }
    }
    if (inv_freq_f64) inv_freq_f64[i] = out;
    if (inv_freq_f32) inv_freq_f32[i] = (float)out;  // RNE under the default mode
  }
  if (attn_factor)
    *attn_factor = (method == YR_ROPE_YARN) ? 0.1 * std::log(factor) + 1.0 : 1.0;
  return YR_OK;
}

// Dynamic NTK ("Arch 03 -- Long Context", NTK-aware slide): at inference time
// the factor follows the sequence, s = current length / training length, and
// the NTK-aware table is built for that s.  Below the training length no
// scaling applies (s = 1, the plain table bit for bit).
extern "C" int yarn_rope_dynamic_ntk_freqs(int head_dim, double base, long long seq_len,
                                           long long original_max_position,
                                           float *inv_freq_f32, double *inv_freq_f64,
                                           double *factor) {
  if (seq_len < 0)
    return yr::fail(YR_ERR_INVALID, "yarn_rope_dynamic_ntk_freqs: seq_len must be >= 0");
  if (original_max_position < 1)
    return yr::fail(YR_ERR_INVALID,
                    "yarn_rope_dynamic_ntk_freqs: original_max_position must be >= 1");
  const double r = (double)seq_len / (double)original_max_position;
  const double s = r > 1.0 ? r : 1.0;
  const int st = yarn_rope_freqs(head_dim, base, s, original_max_position, 1.0, 32.0,
                                 YR_ROPE_NTK, inv_freq_f32, inv_freq_f64, nullptr);
  if (st != YR_OK) return st;
  if (factor) *factor = s;
  return YR_OK;
}
