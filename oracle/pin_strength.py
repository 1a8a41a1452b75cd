"""Pin-strength check for the CPU oracle (test infrastructure; run by hand, not by pytest).

Plants one plausible mistake at a time into a copy of oracle.c (a sign, a tie rule,
a rounding direction, a nibble or swizzle order, a dropped scale, a transposed
operand, ...), builds it, and runs the oracle pin tests against that build through
NVFP4_ORACLE_LIB. Every planted mistake that changes a result must make a pin fail.

    python oracle/pin_strength.py [mutation ...]
"""
import os, subprocess, sys, tempfile, re
ROOT=os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
src=open(os.path.join(ROOT, 'oracle', 'oracle.c')).read()
M = {
 'silu_sign': ('x / (1.0L + expl(-x))', 'x / (1.0L + expl(x))'),
 'silu_tiny_split_lost': ('return rn_bf16_pair(h, h * tanhl(h));', 'return rn_bf16_ld(x / (1.0L + expl(-x)));'),
 'ties_odd': ('int up_is_even = ((j + 1) % 2) == 0;', 'int up_is_even = ((j + 1) % 2) == 1;'),
 'ties_up': ('if (a > mid || (a == mid && up_is_even)) idx = j + 1;', 'if (a >= mid) idx = j + 1;'),
 'gscale_rn': ('while ((double)g * 2688.0 < amax) g = nextafterf(g, INFINITY);', ''),
 'bscale_strict': ('* 6.0 * (double)g >= bmax) return', '* 6.0 * (double)g > bmax) return'),
 'bscale_from1': ('for (int e = 0; e <= 126; ++e)', 'for (int e = 1; e <= 126; ++e)'),
 'nibble_swap': ('(uint8_t)(code[t] | (code[t + 1] << 4))', '(uint8_t)(code[t + 1] | (code[t] << 4))'),
 'swizzle_swap': ('(r & 31) * 16 + ((r >> 5) & 3) * 4', '(r & 31) * 4 + ((r >> 5) & 3) * 16'),
 # bijective alternatives for the order inside a 128 x 4 tile: plain row-major, and
 # the four 32-row groups one after another
 'swizzle_rowmajor': ('(r & 31) * 16 + ((r >> 5) & 3) * 4', '(r & 127) * 4'),
 'swizzle_groupmajor': ('(r & 31) * 16 + ((r >> 5) & 3) * 4', '((r >> 5) & 3) * 128 + (r & 31) * 4'),
 'ue4m3_sub': ('if (E == 0) return ldexp((double)m, -9);', 'if (E == 0) return ldexp((double)m, -10);'),
 'amax_noabs': ('double a = fabs(bf16_to_double(y[i]));', 'double a = bf16_to_double(y[i]);'),
 'y_trunc': ('double p = bf16_to_double(s) * bf16_to_double(up); /* exact: 8 x 8 significant bits */\n  return oracle_rn_bf16(p);',
             'double p = bf16_to_double(s) * bf16_to_double(up);\n  float pf=(float)p; uint32_t uu; memcpy(&uu,&pf,4); return (uint16_t)(uu>>16);'),
 'code_nosign_zero': ('uint8_t sign = signbit(y) ? 8u : 0u;\n  if (s == 0) return sign;', 'uint8_t sign = signbit(y) ? 8u : 0u;\n  if (s == 0) return 0;'),
 'gemm_drop_sw': ('total += (int64_t)dot * (sa[b] * sw[b]);', 'total += (int64_t)dot * (sa[b]);'),
 'gemm_transpose': ('const int8_t* w = W + j * k;', 'const int8_t* w = W + ((j * 7) % n) * k;'),
 'gemm_trunc': ('if (rem > half || (rem == half && (q & 1))) q += 1;', ''),
 'gemm_ties_away': ('if (rem > half || (rem == half && (q & 1))) q += 1;', 'if (rem >= half) q += 1;'),
 'gemm_scale_wrong_block': ('total += (int64_t)dot * (sa[b] * sw[b]);', 'total += (int64_t)dot * (sa[b] * sw[(b+1)%nb]);'),
 'gemm_code_table': ('static const int MAG2[8] = {0, 1, 2, 3, 4, 6, 8, 12};', 'static const int MAG2[8] = {0, 1, 2, 3, 4, 5, 8, 12};'),
 'gemm_nibble': ('A[i * k + c] = (int8_t)q2_of_code((c & 1) ? (byte >> 4) : (byte & 15));', 'A[i * k + c] = (int8_t)q2_of_code((c & 1) ? (byte & 15) : (byte >> 4));'),
 # O11: quantization with a given amax
 'amax_sat_127': ('if (s == 0xFF) s = 126;', 'if (s == 0xFF) s = 127;'),
 'amax_given_abs': ('amax = *amax_given;', 'amax = fabs(*amax_given);'),
 # O12: bias and gated residual in the GEMM epilogue
 'bias_after_round': ('uint16_t d1 = bias ? rn_bf16_sum_exact(neg, P, Ebase, bias[j]) : rn_bf16_exact(neg, P, Ebase);',
                      'uint16_t d1 = bias ? rn_bf16_pair((long double)bf16_to_double(rn_bf16_exact(neg, P, Ebase)), (long double)bf16_to_double(bias[j])) : rn_bf16_exact(neg, P, Ebase);'),
 'gate_on_residual': ('d = rn_bf16_pair((long double)bf16_to_double(res[j]), prod);',
                      'd = rn_bf16_pair(gv * (long double)bf16_to_double(res[j]), (long double)bf16_to_double(d1));'),
 'residual_sign': ('d = rn_bf16_pair((long double)bf16_to_double(res[j]), prod);',
                   'd = rn_bf16_pair(-(long double)bf16_to_double(res[j]), prod);'),
 # O13: adaLN modulation
 'mod_no_one': ('const float mf = 1.0f + (float)bf16_to_double(scale);', 'const float mf = (float)bf16_to_double(scale);'),
 'mod_shift_first': ('const float y = fmaf(xf, mf, (float)bf16_to_double(shift));',
                     'const float y = (xf + (float)bf16_to_double(shift)) * mf;'),
 'mod_unfused': ('const float y = fmaf(xf, mf, (float)bf16_to_double(shift));',
                 'volatile float pm = xf * mf; const float y = pm + (float)bf16_to_double(shift);'),
 'mod_scale_bf16': ('const float mf = 1.0f + (float)bf16_to_double(scale);',
                    'const float mf = (float)bf16_to_double(oracle_rn_bf16(1.0 + bf16_to_double(scale)));'),
 # O14: the SwiGLU pair split and its row maxima
 'pair_swap_gate_up': ('const uint16_t g = d[i * n + 16 * c + e], u = d[i * n + 16 * c + 8 + e];',
                       'const uint16_t u = d[i * n + 16 * c + e], g = d[i * n + 16 * c + 8 + e];'),
 'pair_chunk4': ('const int64_t c = j / 8, e = j % 8;\n      const uint16_t g = d[i * n + 16 * c + e], u = d[i * n + 16 * c + 8 + e];',
                 'const int64_t c = j / 4, e = j % 4;\n      const uint16_t g = d[i * n + 8 * c + e], u = d[i * n + 8 * c + 4 + e];'),
 'pair_ymax_signed': ('const double y = fabs(bf16_to_double(oracle_swiglu_bf16(g, u, tab)));',
                      'const double y = bf16_to_double(oracle_swiglu_bf16(g, u, tab));'),
}
TESTS = ['tests/test_oracle_silu.py', 'tests/test_oracle_quant.py', 'tests/test_oracle_layout.py',
         'tests/test_oracle_gemm.py', 'tests/test_oracle_amax.py', 'tests/test_oracle_epilogue.py',
         'tests/test_oracle_modulate.py', 'tests/test_oracle_swiglu_pair.py']
tmpd=tempfile.mkdtemp()
only=sys.argv[1:]
missing, escaped, caught_n = [], [], 0
for name,(a,b) in M.items():
    if only and name not in only: continue
    if src.count(a) < 1:
        # the mutation no longer applies to the current oracle.c: a failure of this check
        missing.append(name)
        print(f'{name:25s} TARGET MISSING (mutation not applied)', flush=True)
        continue
    msrc=src.replace(a,b)
    cpath=os.path.join(tmpd,name+'.c'); lib=os.path.join(tmpd,name+'.so')
    open(cpath,'w').write(msrc)
    subprocess.run(['gcc','-O2','-fopenmp','-fPIC','-shared','-std=gnu11',cpath,'-o',lib,'-lm'],check=True)
    env=dict(os.environ, NVFP4_ORACLE_LIB=lib)
    r=subprocess.run([sys.executable,'-m','pytest','-x','-q']+TESTS+['-k','not exhaustive_against_decimal or silu'],cwd=ROOT,env=env,capture_output=True,text=True,timeout=900)
    caught = r.returncode!=0
    caught_n += caught
    if not caught: escaped.append(name)
    last=[l for l in r.stdout.splitlines() if 'FAILED' in l or 'passed' in l or 'failed' in l]
    print(f'{name:25s} caught={caught} {last[:1]}',flush=True)
print(f'summary: {caught_n} caught, {len(escaped)} escaped {escaped}, {len(missing)} targets missing {missing}', flush=True)
sys.exit(1 if (escaped or missing) else 0)
