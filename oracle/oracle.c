/*
 * Plain CPU oracle for the batched paged-KV GQA decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source with the HIP library.
 *
 * What it is: single-threaded FP32, no SIMD intrinsics, built without FMA
 * contraction (-ffp-contract=off), one function per operation, in the manner
 * of the plain-C engine "llmc" (section "design conventions": FP32 only,
 * row-major 2-D tensors, FP32 accumulators, one contiguous KV cache per layer
 * of shape [capacity, num_kv_heads * head_dim] with one row appended per
 * token).  The order of operations of one decoder layer follows the
 * "Inference from Scratch" engine summary (its layer op list: QKV
 * projection, RoPE, grouped-query attention, output projection, attention
 * residual, post-attention RMSNorm, SwiGLU MLP, MLP residual; final RMSNorm
 * and the tied embedding / LM head giving FP32 logits; argmax).
 *
 * Attention is the plain definition: scores for every cached token, the
 * maximum, exponentials, their sum, then the weighted sum of V (a two-pass
 * softmax over a contiguous cache).  The paged pool is only ever *gathered*
 * here, into that contiguous cache, to feed the definition; the GPU path
 * must never gather.
 *
 * Readings of points the pages leave open (each one is listed with its
 * reason in the design notes of the repository):
 *   - RoPE pairs element j with element j + D/2 of a head (rotate-half),
 *     with the per-pair rotation of the article's RoPE formula; the angle of
 *     pair j at position p is p * theta^(-2j/D), computed in double, and its
 *     cosine and sine are rounded to FP32.
 *   - RMSNorm is x * (mean(x^2) + eps)^(-1/2) * w, eps inside the root.
 *   - Attention scale 1/sqrt(D); q head h reads kv head h / (Hq/Hkv).
 *   - The new token's K/V is appended (rounded to BF16, nearest-even) before
 *     attention, which then covers positions 0..p inclusive.
 *   - SwiGLU: the packed gate/up weight holds the I gate rows first, then the
 *     I up rows; a = silu(gate) * up with silu(z) = z / (1 + exp(-z)).
 *   - Projections have no bias; the LM head is the embedding matrix itself.
 *   - Argmax returns the lowest index among equal maxima.
 *
 * Pool page layout (the boundary's stated layout, implemented here on its
 * own): a physical page of T tokens holds, as BF16, first the K block, then
 * the V block, both in 16-token tiles: K [slot / 16][kv head][d / 8]
 * [slot % 16][d % 8] (each token's dimensions in chunks of 8) and V
 * [slot / 16][kv head][d][slot % 16] (V transposed within each tile).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- BF16 --- */

/* BF16 -> FP32 is exact: the 16 stored bits are the top half of the FP32. */
float orc_bf16_to_f32(uint16_t h)
{
	uint32_t u = (uint32_t)h << 16;
	float f;
	memcpy(&f, &u, sizeof f);
	return f;
}

/*
 * FP32 -> BF16, round to nearest, ties to even, by its definition: keep the
 * top 16 bits (the value truncated toward zero), look at the 16 discarded
 * bits, and step the kept magnitude up by one BF16 ulp when the discarded
 * part is more than half an ulp, or exactly half and the kept value is odd.
 * A carry out of the mantissa correctly bumps the exponent (up to infinity).
 * NaN stays NaN (quiet bit forced so the top half cannot become infinity).
 */
uint16_t orc_f32_to_bf16(float f)
{
	uint32_t u;
	memcpy(&u, &f, sizeof u);
	if (f != f)
		return (uint16_t)((u >> 16) | 0x0040u);
	uint16_t kept = (uint16_t)(u >> 16);
	uint32_t dropped = u & 0xffffu;
	if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
		kept = (uint16_t)(kept + 1u);
	return kept;
}

void orc_f32_to_bf16_array(const float *x, uint16_t *y, long n)
{
	for (long i = 0; i < n; i++)
		y[i] = orc_f32_to_bf16(x[i]);
}

/* ----------------------------------------------------------- basic ops --- */

/* y = x * (mean(x^2) + eps)^(-1/2) * w   (llmc op "rmsnorm"; BF16 weight). */
void orc_rmsnorm(const float *x, const uint16_t *w, int n, float eps, float *y)
{
	float ss = 0.0f;
	for (int i = 0; i < n; i++)
		ss += x[i] * x[i];
	float ms = ss / (float)n;
	float r = 1.0f / sqrtf(ms + eps);
	for (int i = 0; i < n; i++)
		y[i] = x[i] * r * orc_bf16_to_f32(w[i]);
}

/*
 * y[r] = sum_c W[r][c] * x[c] with W row-major [rows][cols] in BF16 (the
 * Hugging Face [out, in] orientation), FP32 accumulation in index order.
 */
void orc_matvec(const uint16_t *W, int rows, int cols, const float *x, float *y)
{
	for (int r = 0; r < rows; r++) {
		const uint16_t *row = W + (long)r * cols;
		float acc = 0.0f;
		for (int c = 0; c < cols; c++)
			acc += orc_bf16_to_f32(row[c]) * x[c];
		y[r] = acc;
	}
}

/* The RoPE angle's cosine and sine for pair j at position pos, as FP32. */
void orc_rope_cos_sin(int pos, int j, int D, float theta, float *c, float *s)
{
	double inv_freq = pow((double)theta, -2.0 * (double)j / (double)D);
	double ang = (double)pos * inv_freq;
	*c = (float)cos(ang);
	*s = (float)sin(ang);
}

/*
 * Rotate each of `heads` head vectors of length D (stored back to back) by
 * the RoPE angles of position pos.  Pair j is (u_j, u_{j+D/2}):
 *   u_j       <- u_j * cos - u_{j+D/2} * sin
 *   u_{j+D/2} <- u_j * sin + u_{j+D/2} * cos
 */
void orc_rope(float *u, int heads, int D, int pos, float theta)
{
	int half = D / 2;
	for (int h = 0; h < heads; h++) {
		float *v = u + (long)h * D;
		for (int j = 0; j < half; j++) {
			float c, s;
			orc_rope_cos_sin(pos, j, D, theta, &c, &s);
			float a = v[j], b = v[j + half];
			v[j] = a * c - b * s;
			v[j + half] = a * s + b * c;
		}
	}
}

float orc_silu(float z)
{
	return z / (1.0f + expf(-z));
}

/* Index of the largest element; the lowest index wins ties. */
int orc_argmax(const float *v, int n)
{
	int best = 0;
	for (int i = 1; i < n; i++)
		if (v[i] > v[best])
			best = i;
	return best;
}

/* --------------------------------------------------------- attention --- */

/*
 * Grouped-query attention of one sequence over a contiguous cache, by the
 * definition.  q: [hq][D]; kc, vc: [n][hkv * D] (row t = token t); out:
 * [hq][D].  Query head h uses kv head h / (hq / hkv).  For each head:
 *   s_t = (q_h . K_t) * scale,  m = max_t s_t,  e_t = exp(s_t - m),
 *   l = sum_t e_t,              o = (sum_t e_t * V_t) / l.
 * n == 0 gives zeros.
 */
void orc_attention(const float *q, const float *kc, const float *vc, int n,
		   int hq, int hkv, int D, float scale, float *out)
{
	int group = hq / hkv;
	int row = hkv * D;
	float *e = n > 0 ? (float *)malloc(sizeof(float) * (size_t)n) : NULL;
	for (int h = 0; h < hq; h++) {
		int g = h / group;
		const float *qh = q + (long)h * D;
		float *oh = out + (long)h * D;
		if (n == 0) {
			for (int d = 0; d < D; d++)
				oh[d] = 0.0f;
			continue;
		}
		/* pass 1: scores and their maximum */
		float m = -INFINITY;
		for (int t = 0; t < n; t++) {
			const float *kt = kc + (long)t * row + (long)g * D;
			float dot = 0.0f;
			for (int d = 0; d < D; d++)
				dot += qh[d] * kt[d];
			e[t] = dot * scale;
			if (e[t] > m)
				m = e[t];
		}
		/* pass 2: exponentials, their sum, the weighted sum of V */
		float l = 0.0f;
		for (int t = 0; t < n; t++) {
			e[t] = expf(e[t] - m);
			l += e[t];
		}
		for (int d = 0; d < D; d++) {
			float acc = 0.0f;
			for (int t = 0; t < n; t++)
				acc += e[t] * vc[(long)t * row + (long)g * D + d];
			oh[d] = acc / l;
		}
	}
	free(e);
}

/* ------------------------------------------------------------ paging --- */

/*
 * Element offset of (page, K or V, kv head g, slot, d) inside the pool:
 * K at [slot / 16][g][d / 8][slot % 16][d % 8] from the page start, V at
 * [slot / 16][g][d][slot % 16] after the hkv * T * D elements of the K
 * block.
 */
static long pool_offset(long page_elems, int hkv, int T, int D, int page,
			int kv, int g, int slot, int d)
{
	long start = (long)page * page_elems;
	int tile = slot / 16, s = slot % 16;
	if (kv == 0)
		return start + ((((long)tile * hkv + g) * (D / 8) + d / 8) * 16 + s) * 8 + d % 8;
	return start + (long)hkv * T * D + (((long)tile * hkv + g) * D + d) * 16 + s;
}

/*
 * Gather tokens 0..n-1 of one sequence from the pool into a contiguous FP32
 * cache: token t lives in logical page t / T at slot t % T, and the block
 * table row maps the logical page to a physical page.
 */
void orc_pool_gather(const uint16_t *pool, long page_elems, int hkv, int D,
		     int T, const int32_t *bt_row, int n, float *kc, float *vc)
{
	int row = hkv * D;
	for (int t = 0; t < n; t++) {
		int page = bt_row[t / T], slot = t % T;
		for (int g = 0; g < hkv; g++)
			for (int d = 0; d < D; d++) {
				kc[(long)t * row + g * D + d] = orc_bf16_to_f32(
					pool[pool_offset(page_elems, hkv, T, D, page, 0, g, slot, d)]);
				vc[(long)t * row + g * D + d] = orc_bf16_to_f32(
					pool[pool_offset(page_elems, hkv, T, D, page, 1, g, slot, d)]);
			}
	}
}

/* Write one token's BF16 K and V ([hkv][D] each) at position pos. */
void orc_pool_append(uint16_t *pool, long page_elems, int hkv, int D, int T,
		     const int32_t *bt_row, int pos, const uint16_t *k,
		     const uint16_t *v)
{
	int page = bt_row[pos / T], slot = pos % T;
	for (int g = 0; g < hkv; g++)
		for (int d = 0; d < D; d++) {
			pool[pool_offset(page_elems, hkv, T, D, page, 0, g, slot, d)] = k[g * D + d];
			pool[pool_offset(page_elems, hkv, T, D, page, 1, g, slot, d)] = v[g * D + d];
		}
}

/* ------------------------------------------------------------- layer --- */

/*
 * One decoder layer for one sequence whose new token sits at position pos.
 * x [H] is the residual stream (in/out).  kc, vc [cap][hkv*D] hold the
 * cached rows 0..pos-1; row pos is written here (BF16-rounded K and V, as
 * the pool would hold them).  k_new, v_new (optional, [hkv*D]) receive the
 * appended BF16 bits.  Weights are BF16, row-major [out][in]:
 *   w_qkv [(hq + 2 hkv) D][H] (q rows, then k rows, then v rows),
 *   w_o [H][hq D], w_gate_up [2 I][H] (gate rows, then up rows),
 *   w_down [H][I], norms [H].
 * Returns 0, or -1 if pos is outside [0, cap).
 */
int orc_layer_decode(int H, int hq, int hkv, int D, int I, float eps,
		     float theta, const uint16_t *attn_norm,
		     const uint16_t *w_qkv, const uint16_t *w_o,
		     const uint16_t *mlp_norm, const uint16_t *w_gate_up,
		     const uint16_t *w_down, float *x, float *kc, float *vc,
		     int cap, int pos, uint16_t *k_new, uint16_t *v_new,
		     int row_given)
{
	if (pos < 0 || pos >= cap)
		return -1;
	int qd = hq * D, kvd = hkv * D;
	float *xn = (float *)malloc(sizeof(float) * (size_t)H);
	float *qkv = (float *)malloc(sizeof(float) * (size_t)(qd + 2 * kvd));
	float *att = (float *)malloc(sizeof(float) * (size_t)qd);
	float *h1 = (float *)malloc(sizeof(float) * (size_t)H);
	float *gu = (float *)malloc(sizeof(float) * (size_t)(2 * I));
	float *a = (float *)malloc(sizeof(float) * (size_t)I);
	float *y = (float *)malloc(sizeof(float) * (size_t)H);

	/* input RMSNorm, packed QKV projection */
	orc_rmsnorm(x, attn_norm, H, eps, xn);
	orc_matvec(w_qkv, qd + 2 * kvd, H, xn, qkv);
	float *q = qkv, *k = qkv + qd, *v = qkv + qd + kvd;

	/* RoPE on every q head and every k head at the absolute position */
	orc_rope(q, hq, D, pos, theta);
	orc_rope(k, hkv, D, pos, theta);

	/*
	 * append: the cache row holds what the BF16 pool would hold.  With
	 * row_given the caller has already put this token's K/V in row pos
	 * (teacher forcing in tests: the values another implementation wrote)
	 * and the row is left as it is; k_new / v_new still receive this
	 * function's own values.
	 */
	for (int i = 0; i < kvd; i++) {
		uint16_t kb = orc_f32_to_bf16(k[i]), vb = orc_f32_to_bf16(v[i]);
		if (!row_given) {
			kc[(long)pos * kvd + i] = orc_bf16_to_f32(kb);
			vc[(long)pos * kvd + i] = orc_bf16_to_f32(vb);
		}
		if (k_new)
			k_new[i] = kb;
		if (v_new)
			v_new[i] = vb;
	}

	/* attention over positions 0..pos */
	orc_attention(q, kc, vc, pos + 1, hq, hkv, D, 1.0f / sqrtf((float)D), att);

	/* output projection + attention residual */
	orc_matvec(w_o, H, qd, att, y);
	for (int i = 0; i < H; i++)
		h1[i] = x[i] + y[i];

	/* post-attention RMSNorm, SwiGLU MLP, MLP residual */
	orc_rmsnorm(h1, mlp_norm, H, eps, xn);
	orc_matvec(w_gate_up, 2 * I, H, xn, gu);
	for (int i = 0; i < I; i++)
		a[i] = orc_silu(gu[i]) * gu[I + i];
	orc_matvec(w_down, H, I, a, y);
	for (int i = 0; i < H; i++)
		x[i] = h1[i] + y[i];

	free(xn);
	free(qkv);
	free(att);
	free(h1);
	free(gu);
	free(a);
	free(y);
	return 0;
}

/* --------------------------------------------------------- model ends --- */

/* x = E[token] widened to FP32. */
void orc_embed(const uint16_t *E, int H, int token, float *x)
{
	for (int i = 0; i < H; i++)
		x[i] = orc_bf16_to_f32(E[(long)token * H + i]);
}

/*
 * Final RMSNorm and the tied LM head: logits = E * rmsnorm(x) in FP32.
 * Returns the argmax of the logits.
 */
int orc_lm_head(const uint16_t *E, int V, int H, const uint16_t *final_norm,
		float eps, const float *x, float *logits)
{
	float *xn = (float *)malloc(sizeof(float) * (size_t)H);
	orc_rmsnorm(x, final_norm, H, eps, xn);
	orc_matvec(E, V, H, xn, logits);
	free(xn);
	return orc_argmax(logits, V);
}
