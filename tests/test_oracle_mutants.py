"""Planted mistakes in the oracle fail its pins.

Each case below is one plausible slip in ``oracle/oracle.c``: a dropped term, a wrong sign, constant or
index, a transposed operand, a changed order. The test writes a copy of the source with that one text
edit, compiles it with gcc exactly as ``oracle.build()`` does, and runs the pin files that cover the
edited function against the copy (``RL_ORACLE_LIB`` points the oracle's wrapper at it) in a fresh
interpreter. The pins must fail. The unedited oracle passes the same files in the main suite, so each
failure is the planted mistake's doing.

The edits are made on the text (the oracle holds no switches for them); each names an anchor that
occurs once in the source and the text after it to replace, so that an edit which no longer matches the
source fails loudly instead of testing nothing.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

GAE = ["tests/test_oracle_gae.py"]
LOSS = ["tests/test_oracle_loss.py"]
GRAD = ["tests/test_oracle_grad.py"]
VTRACE = ["tests/test_oracle_vtrace.py"]
WAYPOINTS = ["tests/test_oracle_waypoints.py"]
RESPAWN = ["tests/test_oracle_respawn.py"]
ENV = ["tests/test_oracle_env.py"]
HOOK = ["tests/test_oracle_hook.py"]
POLICY = ["tests/test_oracle_policy.py"]

# (name, anchor, old, new, pin files): replace the first `old` after the one occurrence of `anchor` (no
# anchor: `old` itself must occur once).
MUTANTS = [
    # GAE: the definition sum ("Teaching Mario to speedrun", s.6 Better advantages)
    ("gae: bootstrap not cut by the done", "int oracle_gae(", "gamma * v_next * (1.0 - d)", "gamma * v_next", GAE),
    ("gae: lambda dropped from the weights", "int oracle_gae(", "w *= gamma * lambda * (1.0 - d);",
     "w *= gamma * (1.0 - d);", GAE),
    ("gae: later terms not cut by the done", "int oracle_gae(", "w *= gamma * lambda * (1.0 - d);",
     "w *= gamma * lambda;", GAE),
    ("gae: next value taken at t instead of t + 1", "int oracle_gae(",
     "(double)values[(size_t)(k + 1) * N + n]", "(double)values[(size_t)k * N + n]", GAE),
    ("gae: return without the value", "int oracle_gae(", "ret[(size_t)t * N + n] = a + (double)values[(size_t)t * N + n];",
     "ret[(size_t)t * N + n] = a;", GAE),
    # normalisation: population std, eps added to the std
    ("normalize: eps inside the square root", "int oracle_normalize(", "(adv[i] - mean) / (std + eps)",
     "(adv[i] - mean) / sqrt(std * std + eps)", GAE),
    ("normalize: sample std (n - 1)", "int oracle_normalize(", "sqrt(q / (double)n)", "sqrt(q / (double)(n - 1))",
     GAE),
    # the clipped loss ("Don't move too far at once")
    ("loss: max instead of min", "int oracle_ppo_loss(", "double pg = -(s1 < s2 ? s1 : s2);",
     "double pg = -(s1 > s2 ? s1 : s2);", LOSS),
    ("loss: ratio inverted", "int oracle_ppo_loss(", "exp(logp - old_logp[i])", "exp(old_logp[i] - logp)", LOSS),
    ("loss: lower clip bound 1 - 2 eps", "int oracle_ppo_loss(", "ratio < 1.0 - clip_eps ? 1.0 - clip_eps",
     "ratio < 1.0 - 2.0 * clip_eps ? 1.0 - 2.0 * clip_eps", LOSS),
    ("loss: half squared value error", "int oracle_ppo_loss(", "double v = dv * dv;", "double v = 0.5 * dv * dv;",
     LOSS),
    ("loss: entropy sign", "int oracle_ppo_loss(", "ent -= exp(lp) * lp;", "ent += exp(lp) * lp;", LOSS),
    ("loss: entropy added to the total", "int oracle_ppo_loss(", "pg + vf_coef * v - ent_coef * h",
     "pg + vf_coef * v + ent_coef * h", LOSS),
    ("loss: log-sum-exp without the max", "int oracle_ppo_loss(", "double lse = zmax + log(sum);",
     "double lse = log(sum);", LOSS),
    # the loss gradient
    ("grad: entropy term sign", "int oracle_ppo_loss_grad(", "double g_h = ent_coef * pj * (lp + ent);",
     "double g_h = -ent_coef * pj * (lp + ent);", GRAD),
    ("grad: value gradient without the 2", "int oracle_ppo_loss_grad(", "inv * vf_coef * 2.0 * (new_values[i]",
     "inv * vf_coef * (new_values[i]", GRAD),
    ("grad: < for <= at the clip tie", "int oracle_ppo_loss_grad(", "ratio * adv[i] <= clipped * adv[i]",
     "ratio * adv[i] < clipped * adv[i]", GRAD),
    ("grad: one-hot dropped", "int oracle_ppo_loss_grad(", "double onehot = j == a ? 1.0 : 0.0;",
     "double onehot = 0.0;", GRAD),
    ("grad: ratio factor dropped", "int oracle_ppo_loss_grad(", "double g_pg = -adv[i] * ratio * (onehot - pj);",
     "double g_pg = -adv[i] * (onehot - pj);", GRAD),
    # V-trace (IMPALA eq. 1)
    ("vtrace: lambda dropped from c", "int oracle_vtrace(", "double c = lambda * (ratio < c_bar ? ratio : c_bar);",
     "double c = (ratio < c_bar ? ratio : c_bar);", VTRACE),
    ("vtrace: rho dropped from delta", "int oracle_vtrace(", "double delta = rho * (", "double delta = (", VTRACE),
    ("vtrace: V instead of vs in the advantage", "int oracle_vtrace(", "s + 1 < T ? vs[k + N]",
     "s + 1 < T ? (double)values[k + N]", VTRACE),
    ("vtrace: gamma for the masked discount in the product", "int oracle_vtrace(", "w *= g * c;",
     "w *= gamma * c;", VTRACE),
    ("vtrace: c_bar used for the advantage's clip", "int oracle_vtrace(",
     "double rho_pg = ratio < pg_rho_bar ? ratio : pg_rho_bar;", "double rho_pg = ratio < c_bar ? ratio : c_bar;",
     VTRACE),
    # waypoint-path reward (DDNet, Reward Engineering, Version 2)
    ("waypoints: penalty shift 3", None, "#define WP_PENALTY_SHIFT 4", "#define WP_PENALTY_SHIFT 3",
     WAYPOINTS),
    ("waypoints: 128 units per waypoint", None, "#define UNITS_WAYPOINT 256",
     "#define UNITS_WAYPOINT 128", WAYPOINTS),
    ("waypoints: time penalty kept", "/* 12. time:", "if (c->reward_mode == 0) *units -= 1;", "*units -= 1;",
     WAYPOINTS),
    ("waypoints: BFS tries down first", "int oracle_bfs_path(",
     "static const int dc[4] = {1, 0, 0, -1}, dr[4] = {0, -1, 1, 0};",
     "static const int dc[4] = {0, 1, 0, -1}, dr[4] = {1, 0, -1, 0};", WAYPOINTS),
    ("waypoints: a window of 9 after the index", "/* Waypoint-path reward", "#define WP_AHEAD 8",
     "#define WP_AHEAD 9", WAYPOINTS),
    ("waypoints: no clamp for a shortened table", "static int32_t waypoint_units(",
     "if (e->path > len - 1) e->path = len - 1;", "", WAYPOINTS),
    ("waypoints: grace zone 512", None, "#define WP_GRACE 1024", "#define WP_GRACE 512",
     WAYPOINTS),
    # adaptive checkpoint respawn (DDNet, Checkpoint Respawning)
    ("respawn: no starts from the spawn", "static int32_t respawn_choice(",
     "if ((uint32_t)(u1 >> 32) < RESPAWN_START_U32) return 0;", "if (0) return 0;", RESPAWN),
    ("respawn: top half instead of top quarter", "static int32_t respawn_choice(",
     "int32_t q = fill / 4 > 0 ? fill / 4 : 1;", "int32_t q = fill / 2 > 0 ? fill / 2 : 1;", RESPAWN),
    ("respawn: no frontier cap", "static int32_t respawn_choice(",
     "int32_t k = chosen < rs->frontier[m] ? chosen : rs->frontier[m];", "int32_t k = chosen;", RESPAWN),
    ("respawn: every episode raises the frontier", "int oracle_env_step(",
     "if ((ended[n] >> 30) & 1 && outcome > frontier[m])", "if (outcome > frontier[m])", RESPAWN),
    ("respawn: appends in reverse env order", "and those that began at the spawn raise the frontier */",
     "for (int n = 0; n < c->num_envs; ++n) {", "for (int n = c->num_envs - 1; n >= 0; --n) {", RESPAWN),
    ("respawn: second draw reused as the first", "static int32_t respawn_choice(",
     "uint64_t u2 = respawn_draw(rs->seed, rs->counter, n, 2);",
     "uint64_t u2 = respawn_draw(rs->seed, rs->counter, n, 1);", RESPAWN),
    # environment physics and observation (readings pinned by hand-worked episodes)
    ("env: gravity 13", None, "#define GRAVITY 12", "#define GRAVITY 13", ENV),
    ("env: jump speed 121", None, "#define JUMP_V 120", "#define JUMP_V 121", ENV),
    ("env: freeze for 29 ticks", None, "#define FREEZE_TICKS 30", "#define FREEZE_TICKS 29",
     ENV),
    ("env: ground acceleration 4", None, "#define ACC_GROUND 8", "#define ACC_GROUND 4", ENV),
    ("env: frame skip runs past a terminal tick", "int oracle_env_step(",
     "i < c->frame_skip && !terminated && !truncated;", "i < c->frame_skip && !truncated;", ENV),
    ("env: wall snap one short", "/* 5. move along x", "nx = col * TILE - BOX;", "nx = col * TILE - BOX - 1;",
     ENV),
    ("env: outside the map reads as air", "static int tile_at(", "return SOLID;", "return AIR;", ENV),
    ("env: window centre column 22", None, "#define WIN_CX 21", "#define WIN_CX 22", ENV),
    ("env: checkpoint bonus 9", None, "#define UNITS_CHECKPOINT 10240",
     "#define UNITS_CHECKPOINT 9216", ENV),
    ("env: no time penalty", "/* 12. time:", "if (c->reward_mode == 0) *units -= 1;", "", ENV),
    ("env: stack pushed oldest first", "memmove(st + FRAME_DIMS",
     "make_frame(c, &e, st);", "make_frame(c, &e, st + (STACK - 1) * FRAME_DIMS);", ENV),
    ("env: player box not drawn in the pixels", "int oracle_env_obs_pixels(", "v = 255;", "v = 254;", ENV),
    ("env: ceiling snap below the tile", "/* 6. move along y", "ny = (row + 1) * TILE; e->vy = 0;",
     "ny = (row + 1) * TILE + 1; e->vy = 0;", ENV),
    # grapple hook (readings pinned by hand-worked episodes)
    ("hook: 11 ticks of flight", None, "#define HOOK_FLIGHT 10", "#define HOOK_FLIGHT 11", HOOK),
    ("hook: pull 12", None, "#define HOOK_ACCEL 24", "#define HOOK_ACCEL 12", HOOK),
    ("hook: freeze tiles hold the tip", "if (e->hook_phase == HOOK_FLYING) {",
     "if (blocks(tile_at(c, maps, m, floordiv(e->hook_y, TILE), floordiv(e->hook_x, TILE))))",
     "if (tile_at(c, maps, m, floordiv(e->hook_y, TILE), floordiv(e->hook_x, TILE)) != AIR)", HOOK),
    ("hook: fires again while held", "} else if (e->hook_phase == HOOK_IDLE",
     "&& !e->hook_held &&", "&&", HOOK),
    ("hook: floor instead of truncation of the tip speed", "e->hook_vx = (int32_t)",
     "e->hook_vy = (int32_t)((int64_t)aim_dy * HOOK_SPEED / len);",
     "e->hook_vy = (int32_t)floordiv((int32_t)((int64_t)aim_dy * HOOK_SPEED), (int32_t)len);", HOOK),
    # the stand-in inference
    ("policy: Gumbel variate sign", "double oracle_policy_gumbel(", "return -log(-log(u));", "return log(-log(u));",
     POLICY),
    ("policy: bfloat16 truncation instead of rounding", "static float to_bf16(",
     "b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;", "b = b & 0xFFFF0000u;", POLICY),
    ("policy: value row taken for the last logit", "int oracle_policy_forward(",
     "for (int j = 0; j < POLICY_ACTIONS; ++j) {\n            double score",
     "for (int j = 1; j < POLICY_ACTIONS + 1; ++j) {\n            double score", POLICY),
]


def _mutate(text, anchor, old, new):
    anchor = old if anchor is None else anchor
    assert text.count(anchor) == 1, f"anchor {anchor!r} occurs {text.count(anchor)} times"
    start = text.index(anchor)
    pos = text.find(old, start)
    assert pos >= 0, f"{old!r} does not follow {anchor!r}"
    return text[:pos] + new + text[pos + len(old):]


def _run_mutant(args):
    name, anchor, old, new, pins, tmp = args
    src = _mutate(open(SRC).read(), anchor, old, new)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    c_path = os.path.join(tmp, f"{tag}.c")
    so_path = os.path.join(tmp, f"lib{tag}.so")
    with open(c_path, "w") as f:
        f.write(src)
    build = subprocess.run(["gcc", *oracle.GCC_FLAGS, "-w", "-o", so_path, c_path, "-lm"], capture_output=True,
                           text=True)
    if build.returncode != 0:
        return name, None, build.stderr
    env = dict(os.environ, RL_ORACLE_LIB=so_path, PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, "-m", "pytest", *pins, "-x", "-q", "-m", "not gpu"], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    return name, res.returncode, res.stdout[-600:]


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [(*m, tmp) for m in MUTANTS]
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
            results = list(pool.map(_run_mutant, jobs))
    problems = []
    for name, rc, out in results:
        if rc is None:
            problems.append(f"{name}: does not compile\n{out}")
        elif rc == 0:
            problems.append(f"{name}: every pin still passes")
        elif rc != 1:
            problems.append(f"{name}: the pin run ended with status {rc}\n{out}")
    assert not problems, "\n".join(problems)


@pytest.mark.parametrize("m", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_each_edit_matches_the_source(m):
    name, anchor, old, new, pins = m
    text = open(SRC).read()
    assert _mutate(text, anchor, old, new) != text, name
    assert all(os.path.exists(os.path.join(ROOT, p)) for p in pins)
